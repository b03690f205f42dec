"""Host-side model of the dense forward's load schedule (bf16, head dimension 128).

The kernel loads K/V tiles straight into four LDS stages and relies on hand-placed waits:
step m+2 is loaded at the start of phase 2m into the stage of step m-2, and odd phase 2m+1
ends with vmcnt(4) when step m+2 exists, else vmcnt(0), before its barrier. Loads complete
in issue order (four per step and wave). Group 0 reads steps t-1 (P.V) and t (S) in phase
2t, group 1 one phase later. This model checks, for every step count, that each step read
is complete and still in its stage; it also shows that a fixed vmcnt(4) would not be.
"""
import pytest

STAGES = 4


def run_schedule(T: int, tail_wait_all: bool = True) -> None:
    issued = [s for s in (0, 1) if s < T]      # prologue: steps 0 and 1, then a full wait
    done = set(issued)
    owner = {s % STAGES: s for s in issued}
    last_read = {}
    for ph in range(2 * T + 2):
        if ph % 2 == 0:
            s2 = ph // 2 + 2
            if s2 < T:
                prev = owner.get(s2 % STAGES)
                assert prev is None or last_read.get(prev, -1) < ph, f"step {prev} overwritten while in use"
                owner[s2 % STAGES] = s2
                issued.append(s2)
        for group in (0, 1):
            lp = ph - group
            if lp < 0 or lp % 2:
                continue
            t = lp // 2
            for step in ([t - 1] if t >= 1 else []) + [t]:
                if step < T:
                    assert step in done, f"T={T}: step {step} read in phase {ph} before its loads completed"
                    assert owner[step % STAGES] == step
                    last_read[step] = ph
        if ph % 2 == 1:
            m = ph // 2
            newer = 1 if (m + 2 < T or not tail_wait_all) else 0    # vmcnt(4) or vmcnt(0)
            done |= set(issued[:len(issued) - newer] if newer else issued)


@pytest.mark.parametrize("T", range(1, 25))
def test_every_step_is_complete_and_in_place_when_read(T):
    run_schedule(T)


def test_a_fixed_vmcnt4_would_leave_tail_tiles_in_flight():
    with pytest.raises(AssertionError):
        for T in range(1, 25):
            run_schedule(T, tail_wait_all=False)
