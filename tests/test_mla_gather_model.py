"""Host model of the tuned attention kernel's index-list handling, with bounds checks (CPU only).

The 128-head attention kernel (sparse_attention_06_amd/csrc/mla.hip, mla_mfma_kernel) gathers
latent rows straight from HBM into LDS by row id. A wrong row id there is a GPU memory fault, so
this file restates, step for step, how one (row, split) workgroup turns its index list into the
row ids of its gathers, and asserts on the CPU that every address it would load lies inside the
cache, for the inputs that make it take every branch:

  split range   e_begin = split * per, e_end = min(k, e_begin + per); chunks of 2048 entries
  set check     the list is filtered for repeats unless its visible entries (0 <= j <= t) run
                strictly ascending from entry 0 up to e_end
  resolve       entry e -> page_table[seq, j / 64] * 64 + j % 64 if j is visible, j / 64 < ld_pt and
                the page id lies in [0, num_pages); else -1
  repeat filter an entry whose position an earlier entry of the row holds becomes -1
  tile masks    per tile of 32 entries (the tail past the chunk counts as -1): the mask of entries
                >= 0; in a tile with a nonzero mask every -1 takes the tile's first valid row id
  tile loop     only tiles whose mask is nonzero (active tiles) are gathered and computed: the
                first two active tiles are issued up front, active tile j + 2 during active tile
                j's PV product; the entries of the next tile are read one iteration ahead
  gather        wave w (0..3), lane l (0..63): latent loads of tile rows 4i + w (i = 0..7) at
                row * 1152 + 16 l, and the rope load of tile row 8w + l / 8 at row * 1152 + 1024 +
                16 ((l % 8) ^ ((8w + l / 8) / 2 % 8))

Checked: every load's 16 bytes lie in [0, num_pages * 64 * 1152); the list reads stay inside the
chunk's 2048 LDS entries; every key the softmax keeps (mask bit set) is a visible, valid position
listed for the first time in the row; the union over splits of kept positions is exactly the set
the oracle attends (the listed visible positions with a valid page).
"""
import numpy as np
import pytest

PAGE = 64
ROW_BYTES = 1152
NK = 32            # positions per tile
LIST_CAP = 2048    # resolved entries per chunk
STAGE_PAGES = 2048 # page-table entries the staged prologue copies to LDS
NBUF = 3           # tile buffers: two tiles in flight


def pick_splits(rows, k):
    s = 1
    while rows * s < 256 and (k // (s * 2)) >= 4 * NK:
        s *= 2
    return s


def needs_dedupe(row, t, e_end):
    for e in range(1, e_end):
        c, p = int(row[e]), int(row[e - 1])
        vc, vp = 0 <= c <= t, 0 <= p <= t
        if vc and not (vp and p < c):
            return True
    return False


def model_workgroup(row, t, seq, page_table, num_pages, k, splits, sp, check_page=True):
    """Row ids gathered and keys kept by split `sp` of one row; asserts the kernel's bounds.
    check_page=False drops the resolve's page-id range check (a planted mistake)."""
    ld_pt = page_table.shape[1]
    per = ((k + splits - 1) // splits + NK - 1) // NK * NK if splits > 1 else k
    e_begin = sp * per
    e_end = min(k, e_begin + per)
    cache_bytes = num_pages * PAGE * ROW_BYTES
    dedupe = needs_dedupe(row, t, e_end)
    # staged prologue: the index row [0, e_end) and the page-table entries a visible position can
    # use ([0, n_pt)) are copied to LDS first, when they fit; the resolve then reads only those
    n_pt = min(ld_pt, t // PAGE + 1) if (seq >= 0 and t >= 0) else 0
    staged = e_end <= LIST_CAP and n_pt <= STAGE_PAGES
    if staged:
        assert e_end <= LIST_CAP and 4 * (LIST_CAP + STAGE_PAGES) <= 45056
        st_raw = [int(row[e]) for e in range(e_end)]
        st_pt = [int(page_table[seq, p]) for p in range(n_pt)]
    kept = []
    for cb in range(e_begin, e_end, LIST_CAP):
        ce = min(e_end, cb + LIST_CAP)
        n_list = ce - cb
        lst = np.full(LIST_CAP, -(10 ** 9), np.int64)   # stale LDS: never a valid row id
        for e in range(cb, ce):
            if staged:
                assert cb == e_begin and 0 <= e < e_end
                j = st_raw[e]
                vis = 0 <= j <= t and j // PAGE < n_pt
                if vis:
                    assert 0 <= j // PAGE < len(st_pt)
                pg = st_pt[j // PAGE] if vis else -1
            else:
                j = int(row[e])
                vis = seq >= 0 and 0 <= j <= t and j // PAGE < ld_pt
                pg = int(page_table[seq, j // PAGE]) if vis else -1
            ok = 0 <= pg < num_pages if check_page else pg >= 0
            lst[e - cb] = pg * PAGE + j % PAGE if ok else -1
        if dedupe:
            seen = {int(row[e]) for e in range(cb) if 0 <= int(row[e]) <= t}
            for e in range(cb, ce):
                j = int(row[e])
                if lst[e - cb] >= 0 and 0 <= j <= t:
                    if j in seen:
                        lst[e - cb] = -1
                    seen.add(j)
        ntiles = (n_list + NK - 1) // NK
        assert ntiles * NK <= LIST_CAP
        tmask = np.zeros(ntiles, np.int64)
        for tt in range(ntiles):
            vals = [int(lst[tt * NK + h]) if tt * NK + h < n_list else -1 for h in range(NK)]
            m = sum(1 << h for h, v in enumerate(vals) if v >= 0)
            if m:
                sub = vals[(m & -m).bit_length() - 1]
                for h, v in enumerate(vals):
                    if v < 0:
                        lst[tt * NK + h] = sub
            tmask[tt] = m

        def read_entries(tt):
            assert 0 <= tt < ntiles and tt * NK + NK <= LIST_CAP
            return tt, lst[tt * NK: tt * NK + NK].copy(), int(tmask[tt])

        issued = []
        act = [tt for tt in range(ntiles) if tmask[tt]]   # the 64-bit mask of active tiles
        assert ntiles <= 64

        def issue(te):
            tt, ent, m = te
            assert m != 0
            issued.append(tt)
            for w in range(4):
                for lane in range(64):
                    for i in range(8):
                        rid = int(ent[4 * i + w])
                        a = rid * ROW_BYTES + 16 * lane
                        assert 0 <= a and a + 16 <= cache_bytes, (tt, w, lane, rid)
                    slot = 8 * w + lane // 8
                    rid = int(ent[slot])
                    a = rid * ROW_BYTES + 1024 + 16 * ((lane & 7) ^ ((slot >> 1) & 7))
                    assert 0 <= a and a + 16 <= cache_bytes, (tt, w, lane, rid)
            for h in range(NK):
                if (m >> h) & 1:
                    kept.append(cb + tt * NK + h)

        pend = list(act)
        for pt in range(NBUF - 1):
            if pt < len(act):
                issue(read_entries(pend.pop(0)))
        nxt = read_entries(pend.pop(0)) if NBUF - 1 < len(act) else None
        for j in range(len(act)):
            if j + NBUF - 1 < len(act):
                assert nxt is not None and nxt[0] == act[j + NBUF - 1]
                issue(nxt)
                nxt = read_entries(pend.pop(0)) if j + NBUF < len(act) else None
        assert issued == act and not pend
    return kept


def attended_positions(row, t, seq, page_table, num_pages, k, rows_total=1, decode=True):
    """What the kernel attends for the row over all its splits (one list position per kept key):
    the decode entry point splits rows over workgroups, the prefill one does not."""
    splits = pick_splits(rows_total, k) if decode else 1
    kept = []
    for sp in range(splits):
        kept += model_workgroup(row, t, seq, page_table, num_pages, k, splits, sp)
    return kept, splits


def expected_set(row, t, seq, page_table, num_pages):
    ld_pt = page_table.shape[1]
    out = set()
    if seq < 0:
        return out
    for j in row:
        j = int(j)
        if 0 <= j <= t and j // PAGE < ld_pt and 0 <= page_table[seq, j // PAGE] < num_pages:
            out.add(j)
    return out


def _case(rng, t, k, kind, ld_pt, num_pages):
    vis = t + 1
    if kind == "ascending":
        m = min(vis, k)
        lst = np.sort(rng.choice(vis, m, replace=False))
    elif kind == "holes":                 # the fault's shape: short rows, -1 holes, -1 padding
        m = min(vis, k)
        lst = np.sort(rng.choice(vis, m, replace=False))
        lst[rng.integers(0, m, 2)] = -1
    elif kind == "invisible":
        lst = rng.integers(-5, t + 40, min(k, vis + 40))
    elif kind == "repeats":
        base = rng.choice(vis, max(1, min(vis, k // 2)), replace=False)
        lst = np.concatenate([base, rng.choice(base, k - base.size)])
        rng.shuffle(lst)
    elif kind == "all_invalid":
        lst = np.full(k, -1)
    else:
        raise ValueError(kind)
    row = np.full(k, -1, np.int64)
    row[: min(k, lst.size)] = lst[:k]
    return row


@pytest.mark.parametrize("mode", ["decode_1row", "decode_8rows", "prefill"])
@pytest.mark.parametrize("kind", ["ascending", "holes", "invisible", "repeats", "all_invalid"])
@pytest.mark.parametrize("t,k", [(40, 2048), (129, 2048), (3000, 2048), (2047, 2048), (700, 512), (5, 64),
                                 (100, 70), (4500, 4096)])
def test_gather_row_ids_stay_in_bounds(mode, kind, t, k):
    rng = np.random.default_rng(t * 7 + k + len(kind) + len(mode))
    ld_pt = (t + 1 + PAGE - 1) // PAGE + 1
    num_pages = ld_pt + 3
    page_table = rng.permutation(num_pages)[:ld_pt].reshape(1, ld_pt).astype(np.int64)
    if ld_pt > 2:
        page_table[0, -2] = num_pages + 5                                   # a page id past the cache
    if ld_pt > 3:
        page_table[0, 1] = -1                                               # and a negative one
    row = _case(rng, t, k, kind, ld_pt, num_pages)
    rows_total = 8 if mode == "decode_8rows" else 1
    kept, splits = attended_positions(row, t, 0, page_table, num_pages, k, rows_total, mode != "prefill")
    pos = [int(row[e]) for e in kept]
    assert len(pos) == len(set(pos)), "a position attended twice"
    assert set(pos) == expected_set(row, t, 0, page_table, num_pages)


def test_model_catches_a_planted_row_id_past_the_cache():
    """The model's bounds checks fire on a planted mistake: with the resolve's page-id range check
    dropped, an entry on a page id past the cache would be gathered out of bounds."""
    page_table = np.array([[0, 7]], np.int64)     # page 7 does not exist in a 2-page cache
    row = np.array([70] + [-1] * 63, np.int64)
    kept, _ = attended_positions(row, 100, 0, page_table, 2, 64)
    assert kept == [] and expected_set(row, 100, 0, page_table, 2) == set()
    with pytest.raises(AssertionError):
        model_workgroup(row, 100, 0, page_table, 2, 64, 1, 0, check_page=False)


@pytest.mark.parametrize("t,k,decode", [(40, 2048, True), (3000, 2048, False), (4500, 4096, False), (140000, 2048, False)])
def test_row_without_a_page_table_row_gathers_nothing(t, k, decode):
    """A row whose sequence id lies outside the table (seq = -1): nothing is staged or read from
    the page table and no key is kept, in the staged prologue (short lists) and the other one."""
    rng = np.random.default_rng(t + k)
    ld_pt = (t + 1 + PAGE - 1) // PAGE
    page_table = rng.permutation(ld_pt).reshape(1, ld_pt).astype(np.int64)
    row = _case(rng, t, k, "ascending", ld_pt, ld_pt)
    kept, _ = attended_positions(row, t, -1, page_table, ld_pt, k, 1, decode)
    assert kept == []


@pytest.mark.parametrize("t,k,ld_pt", [(3000, 2048, 20), (3000, 2048, 47), (140000, 2048, 2188), (140000, 2048, 3000)])
def test_positions_past_the_page_table_and_rows_over_the_staged_pages(t, k, ld_pt):
    """Page tables narrower than the row (positions on pages past ld_pt are not visible) and rows
    on more pages than the staged prologue copies (t / 64 + 1 > 2048: the resolve reads the page
    table from memory)."""
    rng = np.random.default_rng(ld_pt)
    num_pages = ld_pt + 2
    page_table = rng.permutation(num_pages)[:ld_pt].reshape(1, ld_pt).astype(np.int64)
    row = _case(rng, t, k, "invisible", ld_pt, num_pages)
    for decode in (True, False):
        kept, _ = attended_positions(row, t, 0, page_table, num_pages, k, 1, decode)
        pos = [int(row[e]) for e in kept]
        assert len(pos) == len(set(pos))
        assert set(pos) == expected_set(row, t, 0, page_table, num_pages)
