"""CPU model of the split-role grouped GEMM's pipeline protocol (no GPU).

The kernel's producer waves copy K steps into a ring of three LDS stages and
its consumer waves multiply them. K steps are numbered over all of a
workgroup's tiles (tiles with no K steps issue nothing), with one workgroup
barrier per step: before barrier G the producers have waited for the copies
of step G, and the consumers have finished reading step G - 1, whose stage
the producers refill after the barrier. MXFP8 block scales come either with
each step, into the step's stage, or in batches of four steps of a tile
through a two-slot ring; a batch is started only once the consumers are done
with the batch that last held its slot.

The model replays the producers' rules -- how far ahead they issue (`pump`),
the ring rule, and the copy-counter wait before each barrier -- against a
separate bookkeeping of what each stage and ring slot holds, which copies
are still in flight (they complete in issue order, and a wait for n leaves
at most the last n in flight), and which steps the consumers have read. It
checks, over random and edge-case tile sequences: every step is issued and
both roles pass one barrier per step; at barrier G, step G and its scales
have landed in the places the consumers read; no stage or ring slot is
overwritten before the consumers are done with what it held. Planted
mistakes in the rules (issuing one step further ahead, dropping the ring
rule, a wait that leaves one step too many in flight) must be caught.
"""
import random

import pytest

STAGES = 3
IPP = 4        # operand copies per step and producer wave
SPW = 1        # scale copies per step (or per batch) and producer wave


class Hazard(AssertionError):
    pass


def _run(nks, sbatch, fp8=True, ahead=STAGES - 1, ring_rule=True, wait_steps=STAGES - 2):
    steps = [(ti, kt) for ti, nk in enumerate(nks) for kt in range(nk)]
    total = len(steps)
    batch_of, b = [], -1
    for _, kt in steps:
        if sbatch and kt % 4 == 0:
            b += 1
        batch_of.append(b)

    # ---- the producers' rules, as the kernel states them
    issued, nbatch, bend = 0, 0, [-1, -1]
    # ---- independent bookkeeping
    stage = [None] * STAGES           # step whose operands a stage holds
    ring = [None, None]               # batch whose scales a ring slot holds
    inflight = []                     # copies in issue order: ("op"|"sc"|"bs", step or batch)
    read = set()                      # steps the consumers have finished

    def issue(x):
        nonlocal nbatch
        kt = steps[x][1]
        if fp8 and sbatch and kt % 4 == 0:
            if nbatch > 0:
                bend[(nbatch - 1) & 1] = x - 1
            slot = nbatch & 1
            old = ring[slot]
            if old is not None and any(batch_of[s] == old and s not in read for s in range(total)):
                raise Hazard(f"ring slot {slot} refilled while batch {old} is read")
            ring[slot] = nbatch
            inflight.extend([("bs", nbatch)] * SPW)
            nbatch += 1
        old = stage[x % STAGES]
        if old is not None and old not in read:
            raise Hazard(f"stage {x % STAGES} refilled with step {x} while step {old} is read")
        stage[x % STAGES] = x
        if fp8 and not sbatch:
            inflight.extend([("sc", x)] * SPW)
        inflight.extend([("op", x)] * IPP)

    def pump(done, limit):
        nonlocal issued
        while issued < total and issued <= limit:
            kt = steps[issued][1]
            if fp8 and ring_rule and sbatch and kt % 4 == 0 and bend[nbatch & 1] >= done:
                break
            issue(issued)
            issued += 1

    def wait(n):
        del inflight[:max(0, len(inflight) - n)]

    pump(0, STAGES - 2)
    producer_barriers = 0
    G = 0
    while G < issued:
        wait(wait_steps * IPP if issued - 1 - G >= STAGES - 2 else 0)
        producer_barriers += 1
        # the consumers arrive at barrier G having read step G - 1
        if G > 0:
            read.add(G - 1)
        # after barrier G the consumers read step G and, batched, its batch
        if stage[G % STAGES] != G:
            raise Hazard(f"stage {G % STAGES} holds {stage[G % STAGES]} at barrier {G}")
        if any(c == ("op", G) or c == ("sc", G) for c in inflight):
            raise Hazard(f"step {G} still in flight at its barrier")
        if fp8 and sbatch:
            bt = batch_of[G]
            if ring[bt & 1] != bt or ("bs", bt) in inflight:
                raise Hazard(f"batch {bt} not in ring slot {bt & 1} at barrier {G}")
        pump(G, G + ahead)
        G += 1
    consumer_barriers = total          # one per K step of every tile
    if producer_barriers != consumer_barriers or issued != total:
        raise Hazard(f"barriers {producer_barriers} vs {consumer_barriers}, issued {issued}")


def _random_sequences(seed, n):
    rng = random.Random(seed)
    for _ in range(n):
        yield [rng.choice([0, 1, 1, 2, 3, 4, 5, 8, 9, 13, 32]) for _ in range(rng.randint(0, 12))]


EDGE = [[], [0, 0], [1], [1] * 9, [4, 1, 4], [5, 1, 1, 5], [1, 5, 1, 1, 4], [32, 0, 32], [2, 1]]


@pytest.mark.parametrize("mode", ["bf16", "fp8_per_step", "fp8_batched"])
def test_protocol_holds(mode):
    fp8, sbatch = mode != "bf16", mode == "fp8_batched"
    for nks in EDGE + list(_random_sequences(7, 2000)):
        _run(nks, sbatch, fp8=fp8)


PLANTED = {
    "one_step_further_ahead": dict(ahead=STAGES),
    "no_ring_rule": dict(ring_rule=False),
    "wait_leaves_two_steps": dict(wait_steps=STAGES - 1),
}


@pytest.mark.parametrize("name", sorted(PLANTED))
def test_planted_mistake_is_caught(name):
    caught = False
    for nks in EDGE + list(_random_sequences(8, 500)):
        try:
            _run(nks, True, **PLANTED[name])
        except Hazard:
            caught = True
            break
    assert caught, f"planted mistake '{name}' went unnoticed"
