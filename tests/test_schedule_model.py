"""CPU models of the prefill kernels' LDS protocol and copy addressing.

The prefill kernel (fwd_bf16_pp_kernel, d=128 on 64-key tiles and d=64 on
128-key tiles, the same 16 KiB per tile and the same copies and waits) runs
two groups of four waves one barrier apart; K and V tiles rotate through rings of LDS buffers filled by
asynchronous global->LDS copies that each wave issues for its own rows, waits
on with s_waitcnt vmcnt(N), and publishes with s_barrier.  A tile may only be
read once every wave's copy into its buffer has been waited on before a
barrier the reader has passed, and a buffer may only be refilled after every
wave's last read of it has been retired (lgkmcnt(0), which each barrier
includes) before a barrier the copying wave has passed.  These tests replay
the kernel's program order step by step -- the same buffer choices, lookahead
and waits as the kernel source -- and check both rules for every read, on
short and long sequences, so that a change of the schedule is proven on the
CPU before it runs on a GPU.  The same replay applied to two earlier
schedules (copies waited too late; a work-group with no visible tile copying
tile -1) must fail.

The address models below mirror each copy routine's index arithmetic and
check that every global row it touches lies inside its sequence, that the
LDS swizzles spread every fragment read over all banks, and that every K and
V fragment read of the prefill kernel finds in LDS the (row, chunk) its copy
put there.
"""
import pytest


# ---------------------------------------------------------------------------
# The ping-pong schedule
class Wave:
    def __init__(self, wid, group):
        self.wid, self.group = wid, group
        self.epoch = 0          # barriers passed
        self.vm = []            # outstanding copy instructions, oldest first


def replay(n_kt, nbuf, kahead, vahead, end_wait, mid_wait, waves_per_group=4, guard_empty=True,
           drain_between_tiles=True):
    """Program order of every wave of one work-group of the ping-pong kernel.

    Step j (j = 0 .. n_kt) of a wave: matrix phase reads K_j (buffer j % nbuf)
    and V_{j-1} (buffer (j-1) % nbuf; V_{-1} is the zero-filled buffer);
    copies K_{j+kahead} and V_{j+vahead} (tiles clamped to n_kt - 1); waits
    vmcnt(mid_wait); barrier; softmax phase first reads the early fragments of
    K_{j+1} and V_j; waits vmcnt(end_wait); barrier.  The lagging group starts
    one barrier late and the leading group ends with one extra barrier.  n_kt
    may be a list: the work-group then runs those query tiles one after the
    other (the causal pairing), each tile's reads expecting its own data, with
    a drain (vmcnt 0) and one more barrier between tiles.

    Returns (writes, reads).  A write covers a set of tile rows: a wave's copy
    its own eight rows, or its part of the zero fill of the V_{-1} buffer (a
    plain LDS store retired by the lgkmcnt(0) of the next barrier).  A read
    covers every row and expects a tile label, or None when the values it
    reads are never used.
    """
    waves = [Wave(w, 0 if w < waves_per_group else 1) for w in range(2 * waves_per_group)]
    tiles = n_kt if isinstance(n_kt, (list, tuple)) else [n_kt]
    n_waves = len(waves)
    rows_per_tile = 64
    # rows of a 64-key tile each wave copies (two 4-row slices per wave) and
    # zero-fills (thread t stores 16-byte chunks t, t + 512, ...: rows t / 16
    # and t / 16 + 32)
    copy_rows = {w: frozenset(range(rows_per_tile * w // n_waves, rows_per_tile * (w + 1) // n_waves))
                 for w in range(n_waves)}
    fill_rows = {w: frozenset(r for t in range(64 * w, 64 * w + 64) for r in (t // 16, t // 16 + 32))
                 for w in range(n_waves)}
    writes, reads = [], []

    def kbuf(t):
        return ("K", t % nbuf)

    def vbuf(t):
        return ("V", t % nbuf)

    def write(w, buf, tile, owners, lds_store=False):
        c = {"issuer": w.wid, "owners": owners, "buf": buf, "tile": tile, "issue": w.epoch, "publish": None,
             "idx": len(writes)}
        writes.append(c)
        if lds_store:
            w.lds_pending.append(c)
        else:
            # one copy_tile call: two global_load_lds_dwordx4 instructions (the
            # wave's two 1 KiB slices), each counted by vmcnt
            w.vm.extend([c, c])
        return c

    def wait(w, n):
        # s_waitcnt vmcnt(n): all but the n most recent copy instructions have
        # landed; a copy whose instructions have all landed is published to
        # every wave by this wave's next barrier
        w.vm = w.vm[max(0, len(w.vm) - n):]
        pending = {id(c) for c in w.vm}
        for c in w.issued:
            if c["publish"] is None and id(c) not in pending and c not in w.landed:
                w.landed.append(c)

    def barrier(w):
        for c in w.landed + w.lds_pending:   # barrier() includes lgkmcnt(0)
            if c["publish"] is None:
                c["publish"] = w.epoch + 1
        w.landed, w.lds_pending = [], []
        w.epoch += 1

    def read(w, buf, tile):
        reads.append({"wave": w.wid, "buf": buf, "tile": tile, "epoch": w.epoch})

    for w in waves:
        w.landed, w.lds_pending = [], []
        w.issued = []

        def copy(buf, tile, w=w):
            w.issued.append(write(w, buf, tile, copy_rows[w.wid]))

        for ti, nkt in enumerate(tiles):
            def lab(t, ti=ti):
                return None if t is None else (ti, t)

            def clamp_t(t, nkt=nkt, ti=ti):
                return (ti, min(t, nkt - 1))
            zero = (ti, "zero")
            write(w, vbuf(-1), zero, fill_rows[w.wid], lds_store=True)
            if nkt > 0 or not guard_empty:
                for t in range(kahead):
                    copy(kbuf(t), clamp_t(t))
                for t in range(vahead):
                    copy(vbuf(t), clamp_t(t))
                wait(w, 0)
            barrier(w)
            if w.group == 1:
                barrier(w)
            if nkt > 0 or not guard_empty:
                # preload of step 0
                read(w, kbuf(0), lab(0 if nkt > 0 else None))
                read(w, vbuf(-1), zero)
                for j in range(nkt + 1):
                    read(w, kbuf(j), lab(j if j < nkt else None))
                    read(w, vbuf(j - 1), lab(j - 1) if j >= 1 else zero)
                    copy(kbuf(j + kahead), clamp_t(j + kahead))
                    copy(vbuf(j + vahead), clamp_t(j + vahead))
                    wait(w, mid_wait)
                    barrier(w)
                    # early fragments of step j + 1
                    read(w, kbuf(j + 1), lab((j + 1) if j + 1 < nkt else None))
                    read(w, vbuf(j), lab(j if j < nkt else None))
                    wait(w, end_wait)
                    barrier(w)
            if w.group == 0:
                barrier(w)
            wait(w, 0)
            if ti + 1 < len(tiles) and drain_between_tiles:
                barrier(w)
    epochs = {w.epoch for w in waves}
    assert len(epochs) == 1, f"waves pass different numbers of barriers: {epochs}"
    return writes, reads


def _happens_before(a, b):
    """a is complete before b starts: same wave in program order, or a was
    published by a barrier that b's issuing wave had passed."""
    if a["issuer"] == b["issuer"] and a["idx"] < b["idx"]:
        return True
    return a["publish"] is not None and a["publish"] <= b["issue"]


def check_schedule(writes, reads):
    """Every read sees its tile in every row: among the writes
    into the buffer issued at or before the read's epoch (later ones cannot
    disturb it -- the reader retires its LDS reads before every barrier), none
    of other data may still be in flight, and the last ones in happens-before
    order must all carry the expected tile and be published by then."""
    errors = []
    index = {}
    for c in writes:
        for o in c["owners"]:
            index.setdefault((c["buf"], o), []).append(c)
    owners = {}
    for c in writes:
        owners.setdefault(c["buf"], set()).update(c["owners"])
    for r in reads:
        if r["tile"] is None:
            continue
        for o in sorted(owners.get(r["buf"], ())):
            ws = [c for c in index.get((r["buf"], o), []) if c["issue"] <= r["epoch"]]
            if not ws:
                errors.append(("never written", r, o))
                continue
            for c in ws:
                visible = c["publish"] is not None and c["publish"] <= r["epoch"]
                if c["tile"] != r["tile"] and not visible:
                    errors.append(("write of other data in flight", r, c))
            last_issue = max(c["issue"] for c in ws)
            cand = [c for c in ws if c["publish"] is None or c["publish"] > last_issue or c["issue"] == last_issue]
            last = [c for c in cand if not any(_happens_before(c, d) for d in cand if d is not c)]
            if any(c["tile"] != r["tile"] for c in last):
                errors.append(("stale, overwritten or unordered data", r, [c["tile"] for c in last]))
            elif not all(c["publish"] is not None and c["publish"] <= r["epoch"] for c in last):
                errors.append(("read before the copy was waited and barriered", r, last[0]))
    return errors


# The schedules the kernel source uses, keyed by ring depth: (kahead, vahead,
# end-of-step wait, mid-step wait).  Each step issues 4 copy instructions per
# wave (two for K, two for V), so vmcnt counts are 4 per step.
KERNEL_SCHEDULES = {3: (2, 1, 0, 4), 4: (3, 2, 4, 8)}


@pytest.mark.parametrize("nbuf", sorted(KERNEL_SCHEDULES))
@pytest.mark.parametrize("n_kt", [1, 2, 3, 4, 5, 6, 7, 8, 13, 40])
def test_kernel_schedule_is_race_free(nbuf, n_kt):
    ka, va, end_wait, mid_wait = KERNEL_SCHEDULES[nbuf]
    copies, reads = replay(n_kt, nbuf, ka, va, end_wait, mid_wait)
    assert check_schedule(copies, reads) == []


@pytest.mark.parametrize("nbuf", sorted(KERNEL_SCHEDULES))
@pytest.mark.parametrize("pair", [[5, 12], [12, 5], [1, 1], [0, 7], [7, 0], [4, 4]])
def test_paired_tiles_are_race_free(nbuf, pair):
    """Two query tiles in a row (the causal pairing): the second tile's zero
    fill and first copies must not meet the first tile's last copies."""
    ka, va, end_wait, mid_wait = KERNEL_SCHEDULES[nbuf]
    writes, reads = replay(pair, nbuf, ka, va, end_wait, mid_wait)
    assert check_schedule(writes, reads) == []


def test_paired_tiles_need_the_drain_barrier():
    # four buffers: the last step's copies are still in flight at the tile's
    # final barrier; without the extra barrier the next tile's zero fill races
    # them (n_kt = 5: the last V copy lands in the zero-filled buffer)
    ka, va, end_wait, mid_wait = KERNEL_SCHEDULES[4]
    writes, reads = replay([5, 6], 4, ka, va, end_wait, mid_wait, drain_between_tiles=False)
    assert check_schedule(writes, reads)


@pytest.mark.parametrize("nbuf", sorted(KERNEL_SCHEDULES))
def test_lookahead_limits(nbuf):
    """A ring of nbuf buffers allows K nbuf-1 tiles and V nbuf-2 tiles ahead:
    one more and a copy overwrites a tile the lagging group still reads."""
    ka, va, end_wait, mid_wait = KERNEL_SCHEDULES[nbuf]
    assert ka == nbuf - 1 and va == nbuf - 2
    for bad in ((ka + 1, va), (ka, va + 1)):
        copies, reads = replay(9, nbuf, bad[0], bad[1], end_wait, mid_wait)
        assert check_schedule(copies, reads), bad


def test_waiting_only_for_older_copies_at_step_end_races():
    """The three-buffer schedule needs every copy of a step waited (vmcnt 0)
    before the barrier that ends the step: the other group reads the next
    tiles' early fragments right after it.  Waiting only for the previous
    step's copies there (vmcnt 4) lets a read race its copy."""
    copies, reads = replay(8, 3, 2, 1, 4, 4)
    errs = check_schedule(copies, reads)
    assert errs and any("waited" in e[0] for e in errs)


def test_four_buffer_ring_needs_its_step_end_wait():
    copies, reads = replay(8, 4, 3, 2, 8, 8)
    assert check_schedule(copies, reads)


def test_empty_work_group_copies_nothing():
    """A work-group with no visible tile (n_kt = 0) must issue no copy: the
    clamp min(t, n_kt - 1) would address tile -1."""
    for nbuf, (ka, va, end_wait, mid_wait) in KERNEL_SCHEDULES.items():
        writes, _ = replay(0, nbuf, ka, va, end_wait, mid_wait)
        assert all(c["tile"][1] != -1 for c in writes)
        writes, _ = replay(0, nbuf, ka, va, end_wait, mid_wait, guard_empty=False)
        assert any(c["tile"][1] == -1 for c in writes)


# ---------------------------------------------------------------------------
# The software-pipelined schedule: all eight waves in step, one barrier per
# step.  Step j (j = -1 .. n_kt) computes S_{j+1} from K_{j+1} and
# O += P_{j-1} V_{j-1} on the matrix cores while the softmax of S_j runs on the
# vector ALU; it copies V_{j+1} and then K_{j+3}, reads V_j's first fragments at
# its end (for the next step), waits vmcnt(2) (its own V copy landed, its K
# copy may still be in flight) and ends with a barrier.  Before step -1 the
# work-group zero-fills the V_{-1} buffer, copies K_0 and K_1 and waits for
# them; step -1 only computes S_0.
def replay_sp(n_kt, nbuf=3, end_wait=2, v_ahead=1, k_ahead=3, early_v=True, vbufs=None):
    n_waves = 8
    waves = [Wave(w, 0) for w in range(n_waves)]
    copy_rows = {w: frozenset(range(8 * w, 8 * w + 8)) for w in range(n_waves)}
    fill_rows = {w: frozenset(r for t in range(64 * w, 64 * w + 64) for r in (t // 16, t // 16 + 32))
                 for w in range(n_waves)}
    writes, reads = [], []

    def kbuf(t):
        return ("K", t % nbuf)

    def vbuf(t):
        return ("V", t % (vbufs or nbuf))

    for w in waves:
        w.landed, w.lds_pending, w.issued = [], [], []

        def write(buf, tile, owners, lds_store=False, w=w):
            c = {"issuer": w.wid, "owners": owners, "buf": buf, "tile": tile, "issue": w.epoch, "publish": None,
                 "idx": len(writes)}
            writes.append(c)
            if lds_store:
                w.lds_pending.append(c)
            else:
                w.vm.extend([c, c])
                w.issued.append(c)

        def clamp(t):
            return ("tile", min(t, n_kt - 1))

        def wait(n, w=w):
            w.vm = w.vm[max(0, len(w.vm) - n):]
            pending = {id(c) for c in w.vm}
            for c in w.issued:
                if c["publish"] is None and id(c) not in pending and c not in w.landed:
                    w.landed.append(c)

        def barrier(w=w):
            for c in w.landed + w.lds_pending:
                if c["publish"] is None:
                    c["publish"] = w.epoch + 1
            w.landed, w.lds_pending = [], []
            w.epoch += 1

        def read(buf, tile, w=w):
            reads.append({"wave": w.wid, "buf": buf, "tile": tile, "epoch": w.epoch})

        def lab(t, ok):
            return ("tile", t) if ok else None

        write(vbuf(-1), ("zero",), fill_rows[w.wid], lds_store=True)
        if n_kt > 0:
            write(kbuf(0), clamp(0), copy_rows[w.wid])
            write(kbuf(1), clamp(1), copy_rows[w.wid])
            for t in range(v_ahead - 1):   # a deeper V ring starts its first tiles here
                write(vbuf(t), clamp(t), copy_rows[w.wid])
            wait(0)
        barrier()
        if n_kt > 0:
            for j in range(-1, n_kt + 1):
                write(vbuf(j + v_ahead), clamp(j + v_ahead), copy_rows[w.wid])
                write(kbuf(j + k_ahead), clamp(j + k_ahead), copy_rows[w.wid])
                read(kbuf(j + 1), lab(j + 1, j + 1 < n_kt))            # S_{j+1}
                if j >= 0:
                    read(vbuf(j - 1), lab(j - 1, True) if j >= 1 else ("zero",))   # P_{j-1} V_{j-1}
                if early_v:
                    read(vbuf(j), lab(j, 0 <= j < n_kt) if j >= 0 else ("zero",))  # next step's first V fragments
                wait(end_wait)
                barrier()
        wait(0)
    return writes, reads


SP_SCHEDULE = dict(nbuf=3, end_wait=2, v_ahead=1, k_ahead=3)
# a four-deep V ring: V copies two tiles ahead, both copies of a step may be in
# flight at its end (vmcnt 4)
SP_SCHEDULE_V4 = dict(nbuf=3, vbufs=4, end_wait=4, v_ahead=2, k_ahead=3)


@pytest.mark.parametrize("sched", [SP_SCHEDULE, SP_SCHEDULE_V4], ids=["v3", "v4"])
@pytest.mark.parametrize("n_kt", [1, 2, 3, 4, 5, 6, 7, 8, 13, 40])
def test_sp_schedule_is_race_free(n_kt, sched):
    writes, reads = replay_sp(n_kt, **sched)
    assert check_schedule(writes, reads) == []


@pytest.mark.parametrize("bad", [dict(end_wait=4), dict(k_ahead=4), dict(v_ahead=2),
                                 dict(vbufs=4, end_wait=6, v_ahead=2), dict(vbufs=4, end_wait=4, v_ahead=3)])
def test_sp_schedule_variants_race(bad):
    """Waiting only for the previous step's copies lets the early V reads race;
    one tile more of lookahead overwrites a tile still in use."""
    writes, reads = replay_sp(9, **{**SP_SCHEDULE, **bad})
    assert check_schedule(writes, reads)


# ---------------------------------------------------------------------------
# The fused dK/dV backward kernel: four waves; the block's V rows are copied
# once; the Q and dO tiles of iteration t rotate through two buffers.
# Iteration t first issues the copies of tile t+1 into the other buffer (and
# wave 0 loads the tile's LSE and row dots into registers), computes on
# buffer t % 2, waits for all of its loads (vmcnt 0), lets wave 0 store the
# next LSE/row dots into the other buffer, and ends with a barrier.
def replay_bwd(n_it, nbuf=2, end_wait=0, ahead=1):
    n_waves = 4
    waves = [Wave(w, 0) for w in range(n_waves)]
    rows = {w: frozenset(range(8 * w, 8 * w + 8)) for w in range(n_waves)}
    everyone = frozenset(range(32))
    writes, reads = [], []
    for w in waves:
        w.landed, w.lds_pending, w.issued = [], [], []

        def write(buf, tile, owners, lds_store=False, w=w):
            c = {"issuer": w.wid, "owners": owners, "buf": buf, "tile": tile, "issue": w.epoch, "publish": None,
                 "idx": len(writes)}
            writes.append(c)
            if lds_store:
                w.lds_pending.append(c)
            else:
                w.vm.extend([c, c])
                w.issued.append(c)

        def wait(n, w=w):
            w.vm = w.vm[max(0, len(w.vm) - n):]
            pending = {id(c) for c in w.vm}
            for c in w.issued:
                if c["publish"] is None and id(c) not in pending and c not in w.landed:
                    w.landed.append(c)

        def barrier(w=w):
            for c in w.landed + w.lds_pending:
                if c["publish"] is None:
                    c["publish"] = w.epoch + 1
            w.landed, w.lds_pending = [], []
            w.epoch += 1

        def read(buf, tile, w=w):
            reads.append({"wave": w.wid, "buf": buf, "tile": tile, "epoch": w.epoch})

        if n_it > 0:
            write(("V",), ("v",), frozenset(range(128 * w.wid // 4, 128 * (w.wid + 1) // 4)))
            for t in range(ahead):
                if t < n_it:
                    write(("QdO", t % nbuf), ("tile", t), rows[w.wid])
            wait(0)
            if w.wid == 0:
                write(("L", 0), ("tile", 0), everyone, lds_store=True)
        barrier()
        for t in range(n_it):
            if t + ahead < n_it:
                write(("QdO", (t + ahead) % nbuf), ("tile", t + ahead), rows[w.wid])
            read(("QdO", t % nbuf), ("tile", t))
            read(("L", t % nbuf), ("tile", t))
            read(("V",), ("v",))
            wait(end_wait)
            if w.wid == 0 and t + 1 < n_it:
                write(("L", (t + 1) % nbuf), ("tile", t + 1), everyone, lds_store=True)
            barrier()
    return writes, reads


def replay_dq(n_kt, nbuf=3, ahead=2, prologue_wait=0, end_wait=0):
    """The dQ kernel's pipeline: the prologue copies tiles 0 .. ahead-1 and
    waits (vmcnt(prologue_wait)); iteration t copies tile t+ahead into buffer
    (t+ahead) % nbuf, reads tile t+1 (S and dP) and tile t (K^T for dQ),
    waits (vmcnt(end_wait)) and passes a barrier.  Each wave copies 8 of the
    32 rows of every K and V tile."""
    n_waves = 4
    waves = [Wave(w, 0) for w in range(n_waves)]
    rows = {w: frozenset(range(8 * w, 8 * w + 8)) for w in range(n_waves)}
    writes, reads = [], []
    for w in waves:
        w.landed, w.issued = [], []

        def write(buf, tile, owners, w=w):
            c = {"issuer": w.wid, "owners": owners, "buf": buf, "tile": tile, "issue": w.epoch, "publish": None,
                 "idx": len(writes)}
            writes.append(c)
            w.vm.extend([c, c])
            w.issued.append(c)

        def wait(n, w=w):
            w.vm = w.vm[max(0, len(w.vm) - n):]
            pending = {id(c) for c in w.vm}
            for c in w.issued:
                if c["publish"] is None and id(c) not in pending and c not in w.landed:
                    w.landed.append(c)

        def barrier(w=w):
            for c in w.landed:
                if c["publish"] is None:
                    c["publish"] = w.epoch + 1
            w.landed = []
            w.epoch += 1

        def read(buf, tile, w=w):
            reads.append({"wave": w.wid, "buf": buf, "tile": tile, "epoch": w.epoch})

        for t in range(min(ahead, n_kt)):
            write(("KV", t % nbuf), ("tile", t), rows[w.wid])
        if n_kt > 0:
            wait(prologue_wait)
        barrier()
        if n_kt > 0:
            read(("KV", 0), ("tile", 0))
        for t in range(n_kt):
            if t + ahead < n_kt:
                write(("KV", (t + ahead) % nbuf), ("tile", t + ahead), rows[w.wid])
            if t + 1 < n_kt:
                read(("KV", (t + 1) % nbuf), ("tile", t + 1))
            read(("KV", t % nbuf), ("tile", t))
            wait(end_wait)
            barrier()
    return writes, reads


@pytest.mark.parametrize("n_kt", [1, 2, 3, 4, 5, 9, 20])
def test_dq_pipeline_is_race_free(n_kt):
    writes, reads = replay_dq(n_kt)
    assert check_schedule(writes, reads) == []


@pytest.mark.parametrize("bad", [dict(prologue_wait=2), dict(end_wait=2), dict(nbuf=2), dict(ahead=3)])
def test_dq_pipeline_variants_race(bad):
    # a prologue that waits only for tile 0 (tile 1 is read in iteration 0), a
    # step-end wait that lets the next tile's copies run on, two buffers, or
    # copies three tiles ahead into a three-buffer ring all break it
    writes, reads = replay_dq(6, **bad)
    assert check_schedule(writes, reads) != []


@pytest.mark.parametrize("n_it", [1, 2, 3, 4, 7, 20])
def test_bwd_schedule_is_race_free(n_it):
    writes, reads = replay_bwd(n_it)
    assert check_schedule(writes, reads) == []


@pytest.mark.parametrize("bad", [dict(end_wait=2), dict(ahead=2)])
def test_bwd_schedule_variants_race(bad):
    """Leaving the next tile's copies in flight at the barrier, or copying two
    tiles ahead into a ring of two, lets a read race its copy."""
    writes, reads = replay_bwd(6, **bad)
    assert check_schedule(writes, reads)


# ---------------------------------------------------------------------------
# Copy addressing: every global row a copy reads lies in [0, kv_len)
def pp_copy_rows(t, n_kt, kv_len, BN=64, waves=8, rows_per_copy=4):
    """Rows read by the ping-pong kernel's copy_tile for tile t: the tile is
    clamped to n_kt - 1; each wave copies rows RPI*c .. RPI*c + RPI-1 for its
    two copies c, and rows past the length re-read the last valid row.
    (d = 128: 64-key tiles, 4 rows per copy; d = 64: 128-key tiles, 8 rows.)"""
    t = min(t, n_kt - 1)
    k0 = t * BN
    rows = []
    for w in range(waves):
        for cpy in range(2):
            for lane_row in range(rows_per_copy):
                r = (2 * w + cpy) * rows_per_copy + lane_row
                row = k0 + r
                if k0 + BN > kv_len:
                    row -= max(0, k0 + r - (kv_len - 1))
                rows.append(row)
    return rows


def n_tiles(kv_len, causal, q0, bm, nq, diag, BN=64):
    kend = kv_len
    if causal:
        kend = min(kend, min(q0 + bm, nq) - 1 + diag + 1)
    return (kend + BN - 1) // BN if kend > 0 else 0


PP_TILES = {128: (64, 4), 64: (128, 8)}  # d -> (keys per tile, rows per 1 KiB copy)


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("nq,nk,kv_len,causal", [
    (1, 1, 1, False), (64, 64, 64, True), (65, 65, 65, True), (300, 300, 300, True), (300, 300, 129, True),
    (200, 5, 5, False), (5, 200, 200, True), (256, 256, 0, True), (300, 100, 100, True), (513, 513, 300, False),
    (77, 300, 300, True),
])
def test_pp_copies_stay_inside_the_sequence(nq, nk, kv_len, causal, d):
    BN, rpc = PP_TILES[d]
    diag = nk - nq
    for q0 in range(0, nq, 256):
        nkt = n_tiles(kv_len, causal, q0, 256, nq, diag, BN)
        if nkt == 0:
            continue  # the kernel issues no copy at all (guarded)
        for t in range(0, nkt + 4):
            rows = pp_copy_rows(t, nkt, kv_len, BN, rows_per_copy=rpc)
            assert len(rows) == BN
            assert min(rows) >= 0 and max(rows) < kv_len, (q0, t, min(rows), max(rows))


def test_pp_copy_without_clamp_leaves_the_sequence():
    # the clamp matters: tile n_kt read unclamped runs past a 100-key sequence
    rows = [64 + r for r in range(64)]
    assert max(rows) >= 100


# ---------------------------------------------------------------------------
# LDS swizzles: bijections that spread each fragment read over all banks
def swz128(r):
    return 4 * (r & 3) + ((r >> 2) & 3)


def swz64(r):
    return 4 * ((r >> 1) & 1) + ((r >> 2) & 3)


def swz_v128(r):
    return 4 * (r & 3)


def swz_v64(r):
    return 4 * ((r >> 1) & 1)


@pytest.mark.parametrize("D,swz", [(128, swz128), (64, swz64), (128, swz_v128), (64, swz_v64)])
def test_swizzles_are_bijections_per_row(D, swz):
    cpr = D // 8
    for r in range(64):
        pos = {c ^ swz(r) for c in range(cpr)}
        assert pos == set(range(cpr)), r


def _banks(byte_addrs):
    # 64 banks of 4 bytes; a 16-byte access touches 4 consecutive banks
    out = []
    for a in byte_addrs:
        out.extend(((a // 4) + i) % 64 for i in range(4))
    return out


@pytest.mark.parametrize("D,swz", [(128, swz128), (64, swz64)])
def test_k_fragment_reads_cover_all_banks(D, swz):
    """ds_read_b128 of K fragments: lane li (row li of the 32-key block), chunk
    2*st + hi.  Every 16-lane quarter of the wave (one LDS cycle) touches each
    of the 64 banks exactly once."""
    for st in range(D // 16):
        for quarter in range(4):
            addrs = []
            for lane in range(16 * quarter, 16 * quarter + 16):
                li, hi = lane & 31, lane >> 5
                chunk = (2 * st + hi) ^ swz(li)
                addrs.append((li * D + chunk * 8) * 2)
            assert sorted(_banks(addrs)) == list(range(64)), (st, quarter)


@pytest.mark.parametrize("D,vswz", [(128, swz_v128), (64, swz_v64)])
def test_v_transposed_reads_cover_all_banks(D, vswz):
    """ds_read_b64_tr_b16 of V: in each half wave, 4 rows x 4 chunks (8 bytes
    per lane) cover the 64 banks once per 32 lanes, for every d-block and
    both reads of a pair (8 rows apart)."""
    for db in range(D // 32):
        for u in range(2):
            for half in range(2):
                addrs = []
                for lane in range(32 * half, 32 * half + 32):
                    hi = lane >> 5
                    tr_r = 4 * hi + ((lane & 15) >> 2)
                    tr_cc = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)
                    tr_in = 4 * (lane & 1)
                    r = 8 * u + tr_r
                    elem = r * D + (((4 * db + tr_cc) ^ vswz(r)) * 8) + tr_in
                    addrs.append(elem * 2)
                banks = []
                for a in addrs:
                    banks.extend(((a // 4) + i) % 64 for i in range(2))
                assert sorted(banks) == list(range(64)), (D, db, u, half)


# ---------------------------------------------------------------------------
# Copy -> fragment-read agreement in the ping-pong kernel, for both head
# dimensions: the LDS tile the sixteen 1 KiB copies build, and the (row,
# chunk) every K and V fragment read then finds there.
def pp_lds_tile(D, is_v):
    """Replays copy_tile's LDS writes: {LDS element offset of a 16-byte chunk:
    (tile row, source chunk)}.  Wave w's copies c = 2w, 2w+1 write LDS bytes
    [1024 c, 1024 c + 1024); lane l writes 16 bytes at 1024 c + 16 l, read
    from row RPI*c + l // CPR, chunk (l % CPR) ^ swizzle(row)."""
    BN, rpi = PP_TILES[D]
    cpr = D // 8
    swz = (swz_v128 if D == 128 else swz_v64) if is_v else (swz128 if D == 128 else swz64)
    tile = {}
    for c in range(BN // rpi):
        for lane in range(64):
            row = rpi * c + lane // cpr
            elem = (1024 * c + 16 * lane) // 2
            assert elem not in tile
            tile[elem] = (row, (lane % cpr) ^ swz(row))
    assert len(tile) == BN * cpr
    return tile


@pytest.mark.parametrize("D", [128, 64])
def test_pp_k_reads_find_their_rows(D):
    BN, _ = PP_TILES[D]
    swz = swz128 if D == 128 else swz64
    tile = pp_lds_tile(D, False)
    for kb in range(BN // 32):
        for st in range(D // 16):
            for lane in range(64):
                li, hi = lane & 31, lane >> 5
                off = li * D + (((2 * st + hi) ^ swz(li)) * 8) + kb * 32 * D
                assert tile[off] == (32 * kb + li, 2 * st + hi), (D, kb, st, lane)


@pytest.mark.parametrize("D", [128, 64])
def test_pp_v_reads_find_their_rows(D):
    BN, _ = PP_TILES[D]
    vswz = swz_v128 if D == 128 else swz_v64
    tile = pp_lds_tile(D, True)
    for sl in range(BN // 16):
        for db in range(D // 32):
            for u in range(2):
                for lane in range(64):
                    hi = lane >> 5
                    tr_r = 4 * hi + ((lane & 15) >> 2)
                    tr_cc = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)
                    tr_in = 4 * (lane & 1)
                    off = tr_r * D + (((4 * db + tr_cc) ^ vswz(tr_r)) * 8) + tr_in + 16 * sl * D + 8 * u * D
                    base = off - tr_in  # the 16-byte chunk the 8 bytes lie in
                    assert tile[base] == (16 * sl + 8 * u + tr_r, 4 * db + tr_cc), (D, sl, db, u, lane)


def test_pp_v_read_with_a_row_dependent_swizzle_misses():
    # planted mistake: swz64 (which depends on row bit 3) for d = 64 V tiles
    # breaks the constant per-lane offsets of the second read of a pair
    D = 64
    tile = {}
    for c in range(16):
        for lane in range(64):
            row = 8 * c + lane // 8
            tile[(1024 * c + 16 * lane) // 2] = (row, (lane % 8) ^ swz64(row))
    bad = 0
    for lane in range(64):
        hi = lane >> 5
        tr_r = 4 * hi + ((lane & 15) >> 2)
        tr_cc = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)
        off = tr_r * D + ((tr_cc ^ swz64(tr_r)) * 8) + 8 * D
        bad += tile[off] != (8 + tr_r, tr_cc)
    assert bad > 0


# ---------------------------------------------------------------------------
# Work-group -> (batch, query head) in the forward and dQ kernels: a
# permutation of each query-tile slot's B*Hq work-groups that puts the g query
# heads of a KV head on one XCD (round-robin dispatch: XCD = block index mod 8)
def xcd_grouped_head(j, B, Hq, Hkv):
    g = Hq // Hkv
    if g == 1 or (B * Hkv) % 8 != 0:
        return j
    x, c = j & 7, j >> 3
    group = x + 8 * (c // g)
    b, hk = group // Hkv, group % Hkv
    return b * Hq + hk * g + c % g


@pytest.mark.parametrize("B,Hq,Hkv", [(4, 32, 8), (1, 32, 8), (2, 64, 8), (8, 8, 1), (1, 32, 32), (3, 32, 8),
                                      (2, 16, 4), (1, 8, 2), (16, 64, 1)])
def test_head_mapping_is_a_permutation_grouped_by_xcd(B, Hq, Hkv):
    bh_count = B * Hq
    for slot in range(3):
        heads = []
        for j in range(bh_count):
            block = slot * bh_count + j
            bh = xcd_grouped_head(block % bh_count, B, Hq, Hkv)
            heads.append(bh)
            g = Hq // Hkv
            if g > 1 and (B * Hkv) % 8 == 0:
                b, hq = divmod(bh, Hq)
                kv_group = b * Hkv + hq // g
                assert kv_group % 8 == block % 8, (B, Hq, Hkv, block)  # same XCD for a KV head's heads
        assert sorted(heads) == list(range(bh_count))


# ---------------------------------------------------------------------------
# The 128-row causal kernel's dispatch order (fwd_bf16_kernel): query-tile
# slot s -> tile n-1-s for the first half of the slots, s-half for the rest, so
# that slots s and s+half (one grid-half apart, co-resident on a CU when the
# whole grid fits) carry tiles n-1-s and s, whose causal work adds up to the
# same for every s.
def causal_slot_tile(slot, n):
    half = (n + 1) // 2
    return n - 1 - slot if slot < half else slot - half


@pytest.mark.parametrize("n", list(range(1, 41)))
def test_causal_dispatch_order_is_a_permutation_pairing_heavy_with_light(n):
    tiles = [causal_slot_tile(s, n) for s in range(n)]
    assert sorted(tiles) == list(range(n))
    half = (n + 1) // 2
    # the first half is heaviest first
    assert tiles[:half] == sorted(tiles[:half], reverse=True)
    # slot s and slot s+half hold tiles n-1-s and s: the same sum for every s
    sums = {tiles[s] + tiles[s + half] for s in range(n - half)}
    assert sums <= {n - 1}
