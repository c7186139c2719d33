"""Host-side model of the block-slot chunk loop's schedule (the loop kernel
for grids of 16-unit slices): both wavefront roles must meet the same number
of workgroup barriers, every LDS token block must have landed before it is
read and must not be overwritten while a later slot still reads it, and each
factor set must not be rewritten between its writer's slot and its reader's.

The model restates the kernel's slot sequence: a chunk of nb blocks takes a
start barrier (after the gradient waves load the chunk's operands), one slot
per block and, unless it is the last chunk, a boundary slot; the slot of
block X copies block X + 2 into buffer (X + 2) % 4 at its start and waits for
every copy but those of block X + 2 at its end (the memory counter drains in
issue order); the gradient waves read block X in its slot, the state waves
read block X in the next slot (the boundary slot for a chunk's last block).
"""
import itertools

import pytest

NB = 4  # LDS token blocks
CB = 64  # tokens per block


def schedule(T, C, copies_per_block, stores_per_handover, lead=2, nb=NB, fold=False, grad_fold_barriers=2):
    nblk = (T + CB - 1) // CB
    nbc = C // CB
    nc = (T + C - 1) // C
    nb_last = (T - (nc - 1) * C + CB - 1) // CB
    blocks = [nb_last if c == nc - 1 else nbc for c in range(nc)]
    ops, landed, owner = [], set(), {}
    reads = []  # (slot, block, role)
    fsets = []  # (slot, set, "w" | "r", block)

    def issue(X):
        owner[X % nb] = X
        ops.extend([("copy", X)] * copies_per_block)

    def wait(keep):
        done = ops[:len(ops) - keep] if keep else ops
        for o in done:
            if o[0] == "copy":
                landed.add(o[1])

    def read(slot, X, role):
        assert X in landed, ("not landed", X, role, slot)
        assert owner[X % nb] == X, ("overwritten", X, role, slot)
        reads.append((slot, X, role))

    # state waves
    bar_state = 0
    if fold:
        # the scalar kernels computed in the prologue: the token rows of the
        # first blocks go out first, their coefficients (one copy of the copy
        # wave) only after the gradient waves have written them (barrier after
        # the gate loads, barrier after the scan), then every copy is waited for
        for X in range(min(lead, nblk)):
            owner[X % nb] = X
            ops.extend([("copy", X)] * (copies_per_block - 1))
        bar_state += 1
        ops.extend([("store",)] * stores_per_handover)
        bar_state += 1
        for X in range(min(lead, nblk)):
            ops.append(("copy", X))
        wait(0)
    else:
        for X in range(min(lead, nblk)):
            issue(X)
        ops.extend([("store",)] * stores_per_handover)
        wait(copies_per_block * (min(lead, nblk) - 1))
    bar_state, slot = bar_state + 1, 0
    for c in itertools.count():
        X0, n = c * nbc, blocks[c]
        bar_state += 1  # the chunk's start barrier
        for k in range(n):
            X = X0 + k
            slot += 1
            read(slot, X, "grad")
            fsets.append((slot, X & 1, "w", X))
            if X + lead < nblk:
                issue(X + lead)
            if k > 0:
                read(slot, X - 1, "state")
                fsets.append((slot, (X - 1) & 1, "r", X - 1))
            wait(copies_per_block * max(0, min(X + lead, nblk - 1) - (X + 1)))  # blocks after X + 1 in flight
            bar_state += 1
        slot += 1
        read(slot, X0 + n - 1, "state")
        fsets.append((slot, (X0 + n - 1) & 1, "r", X0 + n - 1))
        if c + 1 == nc:
            break
        ops.extend([("store",)] * stores_per_handover)
        bar_state += 1
    bar_grad = 1 + sum(1 + n for n in blocks) + (nc - 1) + (grad_fold_barriers if fold else 0)
    return nblk, bar_state, bar_grad, reads, fsets


@pytest.mark.parametrize("C", [64, 128, 192, 256, 512, 1024, 2048])
@pytest.mark.parametrize("lead,nb,copies", [(2, 4, 8), (2, 4, 9), (1, 3, 4), (1, 3, 5)])
def test_block_slot_schedule(C, lead, nb, copies):
    """One unit group per workgroup: four blocks, copies two blocks ahead, 8
    copies per state wave (9 for the one that also copies the coefficients);
    two unit groups: three blocks, one ahead, 4 (5) copies."""
    for T in list(range(1, 400)) + [2000, 2048, 4096, 5000, 16384]:
        for stores in (3, 6):  # with the momentum snapshot
            nblk, bs, bg, reads, fsets = schedule(T, C, copies, stores, lead=lead, nb=nb)
            assert bs == bg, (T, C)
            # every block read once by each role, the state after the gradient waves
            grad = {X: s for s, X, r in reads if r == "grad"}
            state = {X: s for s, X, r in reads if r == "state"}
            assert sorted(grad) == sorted(state) == list(range(nblk)), (T, C)
            assert all(state[X] > grad[X] for X in grad), (T, C)
            # a factor set is not rewritten between its write and its read
            for s_r, fs, kind, X in fsets:
                if kind != "r":
                    continue
                s_w = grad[X]
                assert not any(k == "w" and st == fs and s_w < s <= s_r and Y != X
                               for s, st, k, Y in fsets), (T, C, X)


@pytest.mark.parametrize("C", [64, 128, 192, 256])
@pytest.mark.parametrize("lead,nb,copies", [(2, 4, 9), (1, 3, 5)])
def test_block_slot_schedule_folded_scan(C, lead, nb, copies):
    """Calls of at most four chunks, whose prologue computes the scalar
    kernels: the same barrier counts on both roles (two more each), every
    block landed before its first read, with the coefficients of the first
    blocks copied after the scan."""
    for T in range(1, 4 * C + 1):
        nblk, bs, bg, reads, _ = schedule(T, C, copies, 3, lead=lead, nb=nb, fold=True)
        assert bs == bg, (T, C)
        grad = {X: s for s, X, r in reads if r == "grad"}
        assert sorted(grad) == list(range(nblk)), (T, C)
    # a gradient-wave prologue with one barrier fewer than the state waves' is caught
    _, bs, bg, _, _ = schedule(C, C, copies, 3, lead=lead, nb=nb, fold=True, grad_fold_barriers=1)
    assert bs != bg


def test_schedule_model_catches_an_overwrite():
    """The model fails for schedules that would overwrite a block still in
    use: a copy three blocks ahead (into the buffer of block X - 1, which the
    state waves read in the same slot), or two ahead with three buffers."""
    with pytest.raises(AssertionError):
        schedule(1024, 256, 8, 3, lead=3)
    with pytest.raises(AssertionError):
        schedule(1024, 256, 8, 3, lead=2, nb=3)
    schedule(1024, 256, 8, 3)  # the kernel's own schedule passes
