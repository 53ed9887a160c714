"""A host-side model of the LoRA-down kernel's copy schedule (bit_linear_dynamic_amd/csrc/lora_down.hip),
checked on the CPU for every tile geometry the launcher can pick, odd and even tile counts, with and
without the xs output.

The kernel streams x tiles L steps ahead and adapter (A) tiles one step ahead through two rings of LDS
slots, issuing every copy and store itself and waiting with one vmcnt value per step parity (vector
memory operations complete in issue order, so "all but the newest N" is a complete description of a
wait). The model replays one wave's issue order -- prologue x(0), A(0), x(1 .. L-1); then per step A,
then x, then (at the steps that write xs) the xs stores -- and asserts:

* every wait leaves complete every copy of the A and x tiles that its step reads (the step's own
  tiles, and for 32-deep tiles the previous x tile, whose columns the xs stores of an odd step
  combine with its own), and none of those tiles is a dummy copy (one issued past the last tile);
* a copy into a slot is issued only after the last step that reads the slot's previous tile;
* the geometry fits the LDS (160 KiB) and every count stays inside the 6-bit vmcnt field.

The geometry and the wait counts below restate the kernel's LdGeo; a change to one must be made to
the other."""
import pytest

LDS = 160 * 1024


def geometry(RTM: int, NC: int) -> dict:
    BK = 64 if NC == 1 else 32
    CT = 4 * NC
    a_slot = CT * 32 * BK * 2
    x_slot = RTM * 32 * BK * 2 + BK * 4
    x0 = 2 * a_slot + 1024
    cx = (RTM * BK // 16 + 3) // 4
    ca = NC * BK // 16
    xo = cx + 1
    fit = (LDS - x0) // x_slot - 2
    vm = (63 - ca - 2 * RTM) // xo
    L = min(fit, vm, 10)
    return dict(BK=BK, XO=xo, CA=ca, L=L, NX=L + 2, x0=x0, x_slot=x_slot,
                st_even=RTM if BK == 64 else 0, st_odd=RTM)


def replay(RTM: int, NC: int, k_tiles: int, xs: bool, plant: str = ""):
    """plant: a deliberate schedule mistake for the self-test ("stores_without_xs": the waits count
    xs stores that are not issued; "extra_step": the pair loop runs past an odd last tile)."""
    g = geometry(RTM, NC)
    BK, XO, CA, L, NX = g["BK"], g["XO"], g["CA"], g["L"], g["NX"]
    st_even, st_odd = (g["st_even"], g["st_odd"]) if xs else (0, 0)
    w_even, w_odd = (g["st_even"], g["st_odd"]) if (xs or plant == "stores_without_xs") else (0, 0)
    assert L > 1 and g["x0"] + NX * g["x_slot"] <= LDS and CA + L * XO + 2 * RTM < 64
    last_read = {"A": {t: t for t in range(k_tiles)},
                 "X": {t: (t + 1 if (xs and BK == 32 and t % 2 == 0) else t) for t in range(k_tiles)}}
    ops, held = [], {"A": {}, "X": {}}

    def issue(kind, tile, slot, step):
        real = tile < k_tiles
        if real:
            prev = held[kind].get(slot)
            assert prev is None or last_read[kind][prev] < step, (kind, slot, prev, step)
            held[kind][slot] = tile
        ops.extend([(kind if real else "dummy", tile)] * (XO if kind == "X" else CA))

    def wait(n, step, need):
        done = ops[:len(ops) - n]
        for key in need:
            total = ops.count(key)
            assert total > 0, ("never issued", key, step)
            assert done.count(key) == total, ("not complete", key, step, n)

    issue("X", 0, 0, -1)
    issue("A", 0, 0, -1)
    for t in range(1, L):
        issue("X", t, t % NX, -1)
    kt = 0
    while kt + 1 < k_tiles or (plant == "extra_step" and kt < k_tiles):
        wait((L - 1) * XO if kt == 0 else XO + w_odd, kt, [("A", kt), ("X", kt)])
        issue("A", kt + 1, (kt + 1) % 2, kt)
        issue("X", kt + L, (kt + L) % NX, kt)
        ops.extend([("store", kt)] * st_even)
        need = [("A", kt + 1), ("X", kt + 1)] + ([("X", kt)] if xs and BK == 32 else [])
        wait(XO + w_even, kt + 1, need)
        issue("A", kt + 2, (kt + 2) % 2, kt + 1)
        issue("X", kt + 1 + L, (kt + 1 + L) % NX, kt + 1)
        ops.extend([("store", kt + 1)] * st_odd)
        kt += 2
    if kt < k_tiles:  # an odd count of 64-deep tiles: the last step on its own
        assert BK == 64
        wait((L - 1) * XO if kt == 0 else XO + w_odd, kt, [("A", kt), ("X", kt)])


def max_rtm(nc: int) -> int:
    return 6 if nc <= 2 else (5 if nc == 3 else 3)


CASES = [(rtm, nc) for nc in (1, 2, 3, 4) for rtm in range(1, max_rtm(nc) + 1)]


@pytest.mark.parametrize("RTM,NC", CASES)
def test_lora_down_schedule(RTM, NC):
    g = geometry(RTM, NC)
    for xs in (True, False):
        for k_tiles in list(range(1, 14)) + [96, 97, 192, 256, 257]:
            if g["BK"] == 32 and k_tiles % 2:
                continue  # K_pad is a multiple of 64: an even count of 32-deep tiles
            replay(RTM, NC, k_tiles, xs)


def test_model_catches_planted_mistakes():
    """The replay rejects the two schedule mistakes it exists for: counting xs stores in the waits
    when no xs is written, and running a step past an odd last tile."""
    with pytest.raises(AssertionError):
        for k_tiles in (8, 96):
            replay(5, 3, k_tiles, xs=False, plant="stores_without_xs")
    with pytest.raises(AssertionError):
        replay(1, 1, 3, xs=True, plant="extra_step")
