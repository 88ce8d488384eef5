"""The split-K hand-off's counter protocol, checked on a host model.

The persistent and wide kernels hand each output tile to an owner rank with a
bounded wait (gemm.hip, deferred hand-off; wide.hip). One 32-bit counter per
tile holds the arrival count (low 8 bits) and an abandon bit (0x100):

* every rank, including the owner's own workgroup, adds one arrival once its
  partial is stored, and reads back the old value;
* the owner polls until it sees all S arrivals and then finishes the tile; if
  its wait runs out first it sets the abandon bit with a fetch-or and finishes
  only if that fetch-or's old value already shows all S arrivals;
* an arrival that sees the abandon bit and S-1 earlier arrivals finishes the
  tile instead.

In the persistent kernel the owner's own arrival is made by another wave of
its workgroup, so it can land after the owner gave up. The model runs every
order of the S arrivals and the owner's give-up, and checks that exactly one
party finishes each tile. It also checks that a rule excluding the owner's
workgroup from the take-over leaves a tile unfinished.
"""

import itertools

ARRIVALS = 0xFF
ABANDON = 0x100


def take_any(old, S, arriving_rank, owner_rank):
    """The kernels' rule: the S-th arrival after an abandon finishes."""
    return (old & ABANDON) != 0 and (old & ARRIVALS) == S - 1


def take_not_owner(old, S, arriving_rank, owner_rank):
    """A rule that skips the owner's own workgroup."""
    return arriving_rank != owner_rank and take_any(old, S, arriving_rank, owner_rank)


def run(order, give_up_at, S, owner_rank, rule):
    """Finishers of one tile when the ranks arrive in `order` and the owner
    gives up after `give_up_at` arrivals (at S it finds all of them there)."""
    cnt = 0
    finishers = []
    for pos in range(S + 1):
        if pos == give_up_at:
            # the fetch-or; at give_up_at == S it races with the S-th arrival
            # and loses, which ends as a poll that saw all S would
            old, cnt = cnt, cnt | ABANDON
            if (old & ARRIVALS) == S:
                finishers.append("owner")
        if pos < S:
            rank = order[pos]
            old, cnt = cnt, cnt + 1
            if rule(old, S, rank, owner_rank):
                finishers.append(("arrival", rank))
    return finishers


def scenarios(S):
    """Every arrival order (by symmetry only the owner's place matters beyond
    S = 4) and every point at which the owner's wait can run out."""
    owner = 0
    if S <= 4:
        orders = itertools.permutations(range(S))
    else:
        peers = tuple(range(1, S))
        orders = [peers[:p] + (owner,) + peers[p:] for p in range(S)]
    for order in orders:
        for give_up_at in range(S + 1):
            yield order, give_up_at, owner


def test_exactly_one_finisher_for_every_order():
    for S in (2, 3, 4, 8):
        for order, give_up_at, owner in scenarios(S):
            f = run(order, give_up_at, S, owner, take_any)
            assert len(f) == 1, (S, order, give_up_at, f)
            if give_up_at == S:
                assert f == ["owner"]
            else:
                # the abandon came first: the S-th arrival finishes, whoever made it
                assert f == [("arrival", order[-1])], (S, order, give_up_at, f)


def test_excluding_the_owners_workgroup_loses_a_tile():
    """Owner gives up, then its own workgroup's arrival is the last one: a
    rule that skips the owner's workgroup finishes nothing."""
    for S in (2, 4, 8):
        order = tuple(range(1, S)) + (0,)  # the owner's own arrival last
        assert run(order, S - 1, S, 0, take_not_owner) == []
        assert run(order, S - 1, S, 0, take_any) == [("arrival", 0)]
