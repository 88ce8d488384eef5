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


# ---------------------------------------------------------------------------
# Partials held in LDS (persistent kernel, pdefer): the owner's own partial
# is never stored unless the owner gives up. Its give-up must store that
# partial and wait for the stores to complete *before* the abandon bit is
# set, or the rank that takes the tile over could sum a partial that is not
# there yet.
# ---------------------------------------------------------------------------


def run_pdefer(order, give_up_at, S, owner, store_first):
    """Finisher and the partials it could see. Peers store, wait for their
    stores, then arrive; the owner's own arrival is made by another wave of its
    workgroup (its partial stays in LDS). At give_up_at the owner gives up:
    with store_first it stores its held partial (complete) and then sets the
    abandon bit; otherwise the abandon bit goes first and the store lands one
    event later."""
    cnt = 0
    visible = set()
    result = []
    pending_store = False
    events = list(order)
    for pos in range(S + 1):
        if pending_store:  # the owner's late store lands now
            visible.add(owner)
            pending_store = False
        if pos == give_up_at:
            if store_first:
                visible.add(owner)
            old, cnt = cnt, cnt | ABANDON
            if not store_first:
                pending_store = True
            if (old & ARRIVALS) == S:
                result.append(("owner", set(range(S))))  # the owner sums its own from LDS
        if pos < S:
            rank = events[pos]
            if rank != owner:
                visible.add(rank)  # a peer's stores complete before its arrival
            old, cnt = cnt, cnt + 1
            if take_any(old, S, rank, owner):
                result.append((("arrival", rank), set(visible)))
    return result


def test_pdefer_give_up_stores_before_abandon():
    for S in (2, 4, 8):
        for order, give_up_at, owner in scenarios(S):
            res = run_pdefer(order, give_up_at, S, owner, store_first=True)
            assert len(res) == 1, (S, order, give_up_at, res)
            who, seen = res[0]
            assert seen == set(range(S)), (S, order, give_up_at, who, seen)


def test_pdefer_abandon_before_store_loses_a_partial():
    """The planted wrong order: the abandon bit set before the owner's held
    partial is stored. Some order then lets the take-over sum without it."""
    bad = 0
    for S in (2, 4):
        for order, give_up_at, owner in scenarios(S):
            for who, seen in run_pdefer(order, give_up_at, S, owner, store_first=False):
                if who != "owner" and owner not in seen:
                    bad += 1
    assert bad > 0


# ---------------------------------------------------------------------------
# Wide kernel: each wave column's owner makes its own arrival first, then
# waits (bounded) and may give up; peers only arrive. Every interleaving of
# the owner's arrival, its optional give-up after it, and the peers' arrivals
# must leave exactly one finisher.
# ---------------------------------------------------------------------------


def run_wide(order, give_up_after, S, owner):
    """order: the S arrivals in time order (the owner's among them);
    give_up_after: number of arrivals after which the owner gives up (None:
    never; it must come after the owner's own arrival)."""
    cnt = 0
    finishers = []
    owner_done = False
    owner_arrived = False
    for pos in range(S + 1):
        if give_up_after is not None and pos == give_up_after and owner_arrived and not owner_done:
            old, cnt = cnt, cnt | ABANDON
            if (old & ARRIVALS) == S:
                finishers.append("owner")
            owner_done = True
        if pos < S:
            rank = order[pos]
            old, cnt = cnt, cnt + 1
            if rank == owner:
                owner_arrived = True
                if (old & ARRIVALS) == S - 1:  # the others were all here already
                    finishers.append("owner")
                    owner_done = True
            elif (old & ABANDON) and (old & ARRIVALS) == S - 1:
                finishers.append(("arrival", rank))
    if not owner_done and (cnt & ARRIVALS) == S:
        finishers.append("owner")  # the poll sees all S arrivals
    return finishers


def test_wide_owner_arrives_first_exactly_one_finisher():
    for S in (2, 3, 4, 8):
        for order, _, owner in scenarios(S):
            p_owner = order.index(owner)
            for give_up_after in [None] + list(range(p_owner + 1, S + 1)):
                f = run_wide(order, give_up_after, S, owner)
                assert len(f) == 1, (S, order, give_up_after, f)


# ---------------------------------------------------------------------------
# Mailbox hand-off (the persistent kernel's alternative path): peers store
# tagged partials, wait for them, then arrive; the owner polls the tagged
# data itself, finishes, and only then arrives. A give-up is an arrival with
# the abandon bit (one atomic add of 1 + ABANDON). Whoever's arrival brings
# the count to S resets the counter; if the abandon bit is set and that is not
# the owner, it finishes the tile. Every order of the S-1 peer arrivals and
# the owner's (normal or give-up) arrival must give exactly one finisher and
# exactly one reset, and a taker must see every partial.
# ---------------------------------------------------------------------------


def run_mailbox(peer_order, owner_pos, gives_up, S):
    """peer_order: the S-1 peers' arrival order; owner_pos: how many peer
    arrivals precede the owner's; gives_up: the owner's wait runs out (its
    data poll did not see every tag) instead of finishing first."""
    cnt = 0
    finishers, resets = [], 0
    visible = set()
    owner = 0
    events = list(peer_order[:owner_pos]) + ["owner"] + list(peer_order[owner_pos:])
    for ev in events:
        if ev == "owner":
            if gives_up:
                visible.add(owner)  # its held partial is stored and complete first
                old, cnt = cnt, cnt + 1 + ABANDON
                if (old & ARRIVALS) == S - 1:
                    finishers.append(("owner", set(visible)))  # all peers' data is there
                    resets += 1
                    cnt = 0
            else:
                # the data poll saw every peer's tag: all peers stored
                finishers.append(("owner", set(range(S))))
                old, cnt = cnt, cnt + 1
                if (old & ARRIVALS) == S - 1:
                    resets += 1
                    cnt = 0
        else:
            visible.add(ev)  # stores complete before the arrival
            old, cnt = cnt, cnt + 1
            if (old & ARRIVALS) == S - 1:
                if old & ABANDON:
                    finishers.append((("taker", ev), set(visible)))
                resets += 1
                cnt = 0
    return finishers, resets, cnt


def test_mailbox_protocol_one_finisher_one_reset():
    for S in (2, 3, 4, 8):
        peers = tuple(range(1, S))
        orders = itertools.permutations(peers) if S <= 4 else [peers, peers[::-1]]
        for order in orders:
            for owner_pos in range(S):
                # (a normal finish needs every peer's tag, not its arrival:
                # peers store, and may arrive after the owner has finished)
                for gives_up in (False, True):
                    f, resets, cnt = run_mailbox(order, owner_pos, gives_up, S)
                    assert len(f) == 1, (S, order, owner_pos, gives_up, f)
                    assert resets == 1 and cnt == 0, (S, order, owner_pos, gives_up, resets, cnt)
                    assert f[0][1] == set(range(S)), (S, order, owner_pos, gives_up, f)


def test_mailbox_reset_by_owner_race_would_lose_a_tile():
    """The planted alternative: the owner does not arrive and the last peer
    resets. An owner that then gives up finds the count at zero and cannot tell
    'nobody arrived' from 'everyone arrived and reset': the tile is lost."""
    S = 4
    cnt = 0
    for _ in range(S - 1):  # every peer arrives; the last one resets
        old, cnt = cnt, cnt + 1
        if (old & ARRIVALS) == S - 2:
            cnt = 0
    old, cnt = cnt, cnt | ABANDON  # the owner's late give-up
    owner_finishes = (old & ARRIVALS) == S - 1
    assert not owner_finishes and cnt == ABANDON  # nobody finishes; the counter stays dirty
