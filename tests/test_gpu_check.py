"""GPU: pkv_check_metadata flags the contract violations of a step's metadata.

Valid batches (every workload config) give 0; each planted violation sets its
flag; and on seeded random corruptions the device flags equal those of a
row-by-row host check of the same relations (a sequence's rows are its last
q_s positions, a needed table entry names a pool block, a row's slot is its
position's slot under the table)."""
import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu

QSL, QLEN, LEN, SPAN, ENTRY, SRANGE, STABLE = 0x01, 0x02, 0x04, 0x08, 0x10, 0x20, 0x40


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import paged_kv_cache_tables_amd as pkv
    pkv.load_library()
    return torch


def host_flags(m):
    bt, sl, qsl, T, mq, NB, bs, slots = (m[k] for k in ("bt", "sl", "qsl", "T", "mq", "NB", "bs", "slots"))
    S, MB = bt.shape
    f = 0
    if qsl[0] != 0 or qsl[S] != T:
        f |= QSL
    for s in range(S):
        q = int(qsl[s + 1]) - int(qsl[s])
        L = int(sl[s])
        if q < 0:
            f |= QSL
        if q > mq:
            f |= QLEN
        if L < 0 or (q > 0 and L < q):
            f |= LEN
        if L > MB * bs:
            f |= SPAN
        nb = min(-(-L // bs), MB) if L > 0 else 0
        if nb and ((bt[s, :nb] < 0) | (bt[s, :nb] >= NB)).any():
            f |= ENTRY
        if slots is None:
            continue
        for j in range(max(q, 0)):
            i = int(qsl[s]) + j
            if i < 0 or i >= T:
                f |= QSL
                continue
            slot = int(slots[i])
            if slot >= NB * bs:
                f |= SRANGE
            pos = L - q + j
            if pos < 0 or pos // bs >= MB:
                continue
            if slot != int(bt[s, pos // bs]) * bs + pos % bs:
                f |= STABLE
    return f


def meta_of(wl, with_slots=True):
    return dict(bt=wl.block_tables.astype(np.int32).copy(), sl=wl.seq_lens.astype(np.int32).copy(),
                qsl=wl.query_start_loc.astype(np.int32).copy(), T=int(wl.query_start_loc[-1]),
                mq=int(wl.max_query_len), NB=int(wl.num_blocks), bs=int(wl.block_size),
                slots=wl.slot_mapping.astype(np.int64).copy() if with_slots else None)


def device_flags(m):
    import torch
    import paged_kv_cache_tables_amd as pkv
    dev = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return pkv.check_metadata(t(m["bt"]), t(m["sl"]), t(m["qsl"]), m["T"], m["mq"], m["NB"], m["bs"],
                              slot_mapping=None if m["slots"] is None else t(m["slots"]))


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_valid_batches_give_zero(cfg):
    wl = W.make_config(cfg)
    for with_slots in (True, False):
        m = meta_of(wl, with_slots)
        assert host_flags(m) == 0
        assert device_flags(m) == 0, (cfg, with_slots)


def small():
    return W.custom("check", [(5, 1), (40, 3), (33, 33), (1, 1), (70, 1)], 4, 2, 64, 16, seed=3)


PLANTED = [
    ("entry-past-pool", ENTRY, lambda m: m["bt"].__setitem__((1, 0), m["NB"])),
    ("entry-negative", ENTRY, lambda m: m["bt"].__setitem__((2, 1), -5)),
    ("length-below-rows", LEN, lambda m: m["sl"].__setitem__(1, 2)),
    ("length-negative", LEN, lambda m: m["sl"].__setitem__(4, -1)),
    ("length-past-table", SPAN, lambda m: m["sl"].__setitem__(0, m["bt"].shape[1] * m["bs"] + 1)),
    ("query-len-bound", QLEN, lambda m: m.__setitem__("mq", 32)),
    ("slot-past-pool", SRANGE, lambda m: m["slots"].__setitem__(0, m["NB"] * m["bs"])),
    ("slot-off-by-one", STABLE, lambda m: m["slots"].__setitem__(3, m["slots"][3] + 1)),
    ("slot-negative", STABLE, lambda m: m["slots"].__setitem__(5, -1)),
    ("qsl-last", QSL, lambda m: m["qsl"].__setitem__(-1, m["qsl"][-1] - 1)),
    ("qsl-first", QSL, lambda m: m["qsl"].__setitem__(0, 1)),
    ("qsl-decreasing", QSL, lambda m: m["qsl"].__setitem__(2, m["qsl"][3] + 1)),
]


@pytest.mark.parametrize("name,flag,mutate", PLANTED, ids=[p[0] for p in PLANTED])
def test_planted_violation_is_flagged(name, flag, mutate):
    m = meta_of(small())
    assert device_flags(m) == 0
    mutate(m)
    got = device_flags(m)
    assert got & flag, (name, hex(got))
    assert got == host_flags(m), (name, hex(got), hex(host_flags(m)))


def test_random_corruptions_match_the_host_check():
    rng = np.random.default_rng(11)
    base = small()
    for trial in range(40):
        m = meta_of(base, with_slots=bool(trial % 4))
        for _ in range(int(rng.integers(1, 4))):
            kind = int(rng.integers(0, 5))
            S = m["bt"].shape[0]
            s = int(rng.integers(0, S))
            if kind == 0:
                m["bt"][s, int(rng.integers(0, m["bt"].shape[1]))] = int(rng.integers(-3, m["NB"] + 3))
            elif kind == 1:
                m["sl"][s] = int(m["sl"][s]) + int(rng.integers(-4, 5))
            elif kind == 2 and m["slots"] is not None:
                i = int(rng.integers(0, m["T"]))
                m["slots"][i] = int(m["slots"][i]) + int(rng.integers(-20, 21))
            elif kind == 3:
                m["mq"] = int(rng.integers(1, 40))
            elif kind == 4:
                k = int(rng.integers(1, S + 1))
                m["qsl"][k] = max(0, int(m["qsl"][k]) + int(rng.integers(-2, 3)))
        # the metadata check reads slot_mapping rows qsl[s] + j only inside [0, T)
        assert device_flags(m) == host_flags(m), trial
