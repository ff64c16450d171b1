"""GPU checks of the pieces around the block allocator: the copy-on-write block
copy (bit-exact, bf16 and 8-bit pools), and a batch whose block tables and
slots come from the allocator (a cached shared prefix, a fork with
copy-on-write, decode and prefill rows in one call) against the float64 oracle
run over pools built on the host with the oracle's append and a plain block
copy.  The oracle side takes its tables from the allocator model
(oracle.allocator), the GPU side from the library's allocator; the two must agree."""
import hashlib

import numpy as np
import pytest

import oracle
from oracle.allocator import RadixAllocator
import workloads as W
from gpu_harness import compare, to_dev, to_host_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import paged_kv_cache_tables_amd as pkv
    pkv.load_library()
    return torch


@pytest.mark.parametrize("dtype", ["bf16", "u8"])
def test_copy_blocks_bit_exact(gpu, dtype):
    torch = gpu
    import paged_kv_cache_tables_amd as pkv
    print(f"copy blocks {dtype}", flush=True)
    rng = np.random.default_rng(4)
    NB, bs, Hkv, D = 40, 16, 8, 128
    if dtype == "bf16":
        k = rng.integers(0, 1 << 16, size=(NB, bs, Hkv, D), dtype=np.uint16)
        v = rng.integers(0, 1 << 16, size=(NB, bs, Hkv, D), dtype=np.uint16)
        kd = torch.from_numpy(k.view(np.int16)).view(torch.bfloat16).to("cuda:0")
        vd = torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    else:
        k = rng.integers(0, 256, size=(NB, bs, Hkv, D), dtype=np.uint8)
        v = rng.integers(0, 256, size=(NB, bs, Hkv, D), dtype=np.uint8)
        kd, vd = torch.from_numpy(k).to("cuda:0"), torch.from_numpy(v).to("cuda:0")
    src = np.array([3, 7, 7, 12, 39, 5, -1, 50, 9], dtype=np.int32)
    dst = np.array([20, 21, 22, 23, 0, 5, 24, 25, 41], dtype=np.int32)   # 5->5, -1, 50, 41 are skipped
    pkv.kv_copy_blocks(kd, vd, torch.from_numpy(src).to("cuda:0"), torch.from_numpy(dst).to("cuda:0"))
    torch.cuda.synchronize()
    k2, v2 = k.copy(), v.copy()
    for s, d in zip(src, dst):
        if s != d and 0 <= s < NB and 0 <= d < NB:
            k2[d], v2[d] = k[s], v[s]
    got_k = kd.view(torch.int16).cpu().numpy().view(np.uint16) if dtype == "bf16" else kd.cpu().numpy()
    got_v = vd.view(torch.int16).cpu().numpy().view(np.uint16) if dtype == "bf16" else vd.cpu().numpy()
    assert np.array_equal(got_k, k2) and np.array_equal(got_v, v2)


def kv_rows(prefix, Hkv, D):
    """K and V rows (bf16 bits) of the token that ends ``prefix``: a seeded function of the
    whole prefix, so equal prefixes have equal rows, as their cached K/V would."""
    seed = int.from_bytes(hashlib.sha256(np.asarray(prefix, np.int64).tobytes()).digest()[:8], "little")
    r = np.random.default_rng(seed)
    k = W.f32_to_bf16_bits(r.standard_normal((Hkv, D), dtype=np.float32))
    v = W.f32_to_bf16_bits(r.standard_normal((Hkv, D), dtype=np.float32))
    return k, v


def test_allocator_tables_drive_the_attention(gpu):
    torch = gpu
    import paged_kv_cache_tables_amd as pkv
    print("allocator-driven batch", flush=True)
    NB, bs, Hq, Hkv, D = 64, 16, 8, 2, 128
    rng = np.random.default_rng(21)
    system = list(rng.integers(0, 1000, 40))
    prompts = {name: system + list(rng.integers(0, 1000, n)) for name, n in (("r1", 20), ("r2", 10), ("r3", 25))}
    model, native = RadixAllocator(NB, bs), pkv.BlockAllocator(NB, bs)
    k_host = np.full((NB, bs, Hkv, D), W.BF16_QNAN, np.uint16)
    v_host = k_host.copy()
    k_dev = torch.from_numpy(k_host.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    v_dev = torch.from_numpy(v_host.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    tokens = {}

    def both(fn, *args):
        a, b = getattr(model, fn)(*args), getattr(native, fn)(*args)
        assert a == b, (fn, a, b)
        return a

    def write(name, aid, positions):
        """Append the K/V rows of these positions: host pools (oracle append), device pools."""
        nonlocal k_host, v_host
        toks = tokens[name]
        for pos in positions:
            if pos == positions[0] or pos % bs == 0:
                cp = both("prepare_write", aid, pos)
                if cp is not None:
                    s, d = cp
                    k_host[d], v_host[d] = k_host[s], v_host[s]
                    pkv.kv_copy_blocks(k_dev, v_dev, torch.tensor([s], dtype=torch.int32, device="cuda:0"),
                                       torch.tensor([d], dtype=torch.int32, device="cuda:0"))
        rows = [kv_rows(toks[:p + 1], Hkv, D) for p in positions]
        kn = np.stack([r[0] for r in rows]); vn = np.stack([r[1] for r in rows])
        slots = np.array(both("slots", aid, positions[0], len(positions)), dtype=np.int64)
        k_host, v_host = oracle.kv_append(k_host, v_host, kn, vn, slots)
        pkv.kv_append(to_dev(kn, torch.bfloat16), to_dev(vn, torch.bfloat16), to_dev(slots, torch.int64),
                      k_dev, v_dev)

    # r1 and r2 prefill from scratch; r1 finishes and its prefix is cached
    ids = {}
    for name in ("r1", "r2"):
        tokens[name] = prompts[name]
        aid, blocks, pre = both("allocate", prompts[name], len(prompts[name]) + 8)
        assert pre == 0
        ids[name] = aid
        write(name, aid, list(range(len(prompts[name]))))
    both("free", ids.pop("r1"), tokens["r1"])
    # r3 shares the 40-token system prompt: two whole blocks come from the cache
    tokens["r3"] = prompts["r3"]
    aid, blocks, pre = both("allocate", prompts["r3"], len(prompts["r3"]) + 4)
    assert pre == 32
    ids["r3"] = aid
    write("r3", aid, list(range(pre, len(prompts["r3"]))))
    # r2 forks (e.g. a second sample); both branches decode one token: copy-on-write of the
    # shared last block
    fid, _ = both("fork", ids["r2"], len(prompts["r2"]))
    ids["f"] = fid
    tokens["f"] = prompts["r2"] + [777]
    tokens["r2"] = prompts["r2"] + [555]
    n2 = len(prompts["r2"])
    both("extend", fid, n2 + 1)
    write("r2", ids["r2"], [n2])
    write("f", fid, [n2])

    # one attention call: r2 and f decode their new token, r3 its 33 uncached prompt rows as a chunk
    order = [("r2", 1), ("f", 1), ("r3", len(prompts["r3"]) - pre)]
    L = [len(tokens[n]) for n, _ in order]
    qn = [q for _, q in order]
    qsl = np.concatenate([[0], np.cumsum(qn)]).astype(np.int32)
    max_blocks = max(-(-l // bs) for l in L) + 1
    bt = np.full((len(order), max_blocks), -1, np.int32)
    for i, (n, _) in enumerate(order):
        tb = both("table", ids[n])
        bt[i, :len(tb)] = tb
    q = W.f32_to_bf16_bits(rng.standard_normal((int(qsl[-1]), Hq, D), dtype=np.float32))
    scale = float(np.float32(1.0) / np.sqrt(np.float32(D)))
    ref = oracle.paged_attention(q, k_host, v_host, bt, np.array(L, np.int32), qsl, Hkv, scale)
    out = torch.empty((int(qsl[-1]), Hq, D), dtype=torch.bfloat16, device="cuda:0")
    pkv.paged_attention(out, to_dev(q, torch.bfloat16), k_dev, v_dev, to_dev(bt, torch.int32),
                        to_dev(np.array(L, np.int32), torch.int32), to_dev(qsl, torch.int32), scale, max(qn))
    torch.cuda.synchronize()
    # the device pools equal the host ones (appends and the block copy), then the outputs
    assert np.array_equal(k_dev.view(torch.int16).cpu().numpy().view(np.uint16), k_host)
    assert np.array_equal(v_dev.view(torch.int16).cpu().numpy().view(np.uint16), v_host)
    compare(to_host_bits(out), ref, label="allocator-driven")
    # the two branches of the fork differ only in their last token
    assert not np.array_equal(to_host_bits(out)[0], to_host_bits(out)[1])
