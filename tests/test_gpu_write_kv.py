"""GPU checks of the append path (needs a gfx950 GPU).

A decode step first appends the new token's K/V at the slot the host pool
hands out, then attends over the whole cache.  Here sequences are admitted
with a prompt, grown one token at a time in round-robin order (so their pages
interleave in the pool), and every row is written with pkv_write_kv.  The
device pools must equal, byte for byte, a host pool built with the oracle's
byte scatter; decoding over them must match the oracle, and be bitwise equal
to decoding the same logical cache laid out by the generator (different
physical pages, same logical order).
"""

import dataclasses

import numpy as np
import pytest

import oracle
from gpu_helpers import compare, gpu_decode, note, small_config
from synth import make_case
from synth.device import torch_dtype, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_266_amd as pkv

    pkv.lib()
    yield


def _as_torch(a, dtype_name, device):
    import torch

    if dtype_name == "i8":
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)
    if dtype_name == "fp8":
        return torch.from_numpy(np.ascontiguousarray(a)).to(device).view(torch.float8_e4m3fn)
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    return t.view(torch_dtype(dtype_name)).to(device)


@pytest.mark.parametrize("Hq,Hkv,D,qd,kvd,PS,lens", [
    (8, 2, 64, "f16", "f16", 16, (37, 100, 5, 16)),
    (32, 8, 128, "bf16", "bf16", 64, (300, 64, 1, 129)),
    (16, 16, 128, "f16", "i8", 16, (77, 200, 33)),
    (8, 4, 128, "bf16", "i8", 64, (65, 130)),
    (16, 4, 128, "bf16", "fp8", 64, (200, 64, 3)),
    (8, 8, 64, "f16", "fp8", 16, (40, 17)),
])
def test_append_write_then_decode(Hq, Hkv, D, qd, kvd, PS, lens):
    import torch

    import paged_kv_cache_266_amd as pkv

    cfg = small_config(Hq, Hkv, D, qd, kvd, PS, lens)
    case = make_case(cfg, keep_logical=True)
    note(f"write_kv: Hq {Hq} Hkv {Hkv} D {D} {qd}/{kvd} PS {PS} lens {lens}")
    dev = "cuda"
    shape = (cfg.num_pages, Hkv, PS, D)
    kv_t = torch_dtype(kvd)
    i8 = kvd in ("i8", "fp8")            # byte codes with one scale per row
    k_pool = torch.zeros(shape, dtype=torch.uint8 if kvd == "fp8" else kv_t, device=dev).view(kv_t)
    v_pool = torch.zeros(shape, dtype=torch.uint8 if kvd == "fp8" else kv_t, device=dev).view(kv_t)
    k_sc = torch.zeros(shape[:3], dtype=torch.float32, device=dev) if i8 else None
    v_sc = torch.zeros(shape[:3], dtype=torch.float32, device=dev) if i8 else None
    host_k = np.zeros(shape, dtype=(np.uint8 if kvd == "fp8" else np.int8) if i8 else np.uint16)
    host_v = np.zeros_like(host_k)
    host_ks = np.zeros(shape[:3], dtype=np.float32) if i8 else None
    host_vs = np.zeros_like(host_ks) if i8 else None

    def put(b, lo, hi, slots):
        if hi == lo:
            return
        (k_enc, k_s), (v_enc, v_s) = case.logical_k[b], case.logical_v[b]
        kn, vn = k_enc[lo:hi], v_enc[lo:hi]
        pkv.write_kv(_as_torch(kn, kvd, dev), _as_torch(vn, kvd, dev),
                     torch.from_numpy(slots).to(dev), k_pool, v_pool,
                     k_scale_new=None if not i8 else torch.from_numpy(np.ascontiguousarray(k_s[lo:hi])).to(dev),
                     v_scale_new=None if not i8 else torch.from_numpy(np.ascontiguousarray(v_s[lo:hi])).to(dev),
                     k_scale=k_sc, v_scale=v_sc)
        oracle.scatter_rows(host_k, slots, kn)
        oracle.scatter_rows(host_v, slots, vn)
        if i8:
            oracle.scatter_rows(host_ks[..., None], slots, k_s[lo:hi][..., None])
            oracle.scatter_rows(host_vs[..., None], slots, v_s[lo:hi][..., None])

    prompt = [max(n - 40, n // 2) for n in lens]
    with pkv.KVPool(cfg.num_pages, PS) as pool:
        for b, n0 in enumerate(prompt):
            put(b, 0, n0, pool.allocate(b, n0))
        count = list(prompt)
        while any(c < n for c, n in zip(count, lens)):
            for b, n in enumerate(lens):
                if count[b] < n:
                    put(b, count[b], count[b] + 1, pool.append_tokens(b, 1))
                    count[b] += 1
        bt, ctx = pool.block_tables(list(range(len(lens))), cfg.max_blocks)
    torch.cuda.synchronize()

    # the device pools hold exactly the bytes the host scatter put there
    assert np.array_equal(k_pool.cpu().view(torch.uint8 if i8 else torch.int16).numpy().view(host_k.dtype), host_k)
    assert np.array_equal(v_pool.cpu().view(torch.uint8 if i8 else torch.int16).numpy().view(host_v.dtype), host_v)
    if i8:
        assert np.array_equal(k_sc.cpu().numpy(), host_ks)
        assert np.array_equal(v_sc.cpu().numpy(), host_vs)
    assert np.array_equal(ctx, case.context_lens)

    # decode over the written pool: the oracle on the same pool, and the
    # generator's own layout of the same logical cache, bitwise
    written = dataclasses.replace(
        case, block_tables=bt, used_pages=np.arange(cfg.num_pages, dtype=np.int32),
        page_index=np.arange(cfg.num_pages, dtype=np.int32), k_pages=host_k, v_pages=host_v,
        k_scale=host_ks, v_scale=host_vs)
    q = upload(case, dev).q
    out = pkv.paged_attn_decode(q, k_pool, v_pool, torch.from_numpy(bt).to(dev),
                                torch.from_numpy(ctx).to(dev), case.scale,
                                max_context_len=cfg.max_context_len, k_scale=k_sc, v_scale=v_sc)
    torch.cuda.synchronize()
    compare(written, out, "decode over written pool")
    ref_layout = gpu_decode(case)
    assert torch.equal(out.view(torch.int16), ref_layout.view(torch.int16))


@pytest.mark.parametrize("Hkv,D,src,kvd,PS", [
    (8, 128, "bf16", "i8", 64),
    (4, 64, "f16", "i8", 16),
    (8, 128, "bf16", "fp8", 64),
    (2, 64, "f16", "fp8", 16),
    (16, 128, "f16", "fp8", 16),
])
def test_quantise_on_append_matches_oracle(Hkv, D, src, kvd, PS):
    """f16 / bf16 rows written into an int8 / fp8 pool are quantised on the
    device: codes and scales equal, bit for bit, the oracle's quantiser of
    the same (exactly decoded) values, at the right slots."""
    import torch

    import paged_kv_cache_266_amd as pkv
    from synth.make import _to_bits

    note(f"quantise-on-append: Hkv {Hkv} D {D} {src}->{kvd} PS {PS}")
    rng = np.random.default_rng(77)
    n, num_pages = 150, 64
    xs = []
    for _ in range(2):   # K and V
        x = rng.standard_normal((n, Hkv, D)).astype(np.float32) * 2.0
        x[0] = 0.0                          # all-zero rows: the scale floor
        x[1, :, 5] = 300.0                  # outliers
        x[2] *= 1e-6                        # below the floor
        bits = _to_bits(x, src)
        exact = (bits.view(np.float16).astype(np.float32) if src == "f16"
                 else (bits.astype(np.uint32) << 16).view(np.float32))
        xs.append((bits, exact))
    slots = rng.permutation(num_pages * PS)[:n].astype(np.int64)
    dev = "cuda"
    shape = (num_pages, Hkv, PS, D)
    kv_t = torch_dtype(kvd)
    pools = [torch.zeros(shape, dtype=torch.uint8, device=dev).view(kv_t) for _ in range(2)]
    scales = [torch.zeros(shape[:3], dtype=torch.float32, device=dev) for _ in range(2)]
    new = [_as_torch(b, src, dev) for b, _ in xs]
    pkv.write_kv(new[0], new[1], torch.from_numpy(slots).to(dev), pools[0], pools[1],
                 k_scale=scales[0], v_scale=scales[1])
    torch.cuda.synchronize()
    for (bits, exact), pool, sc in zip(xs, pools, scales):
        codes, s = oracle.quantize_rows(exact, kvd)
        want_pool = np.zeros(shape, dtype=np.uint8)
        want_sc = np.zeros(shape[:3], dtype=np.float32)
        oracle.scatter_rows(want_pool, slots, codes.view(np.uint8))
        oracle.scatter_rows(want_sc[..., None], slots, s[..., None])
        got_pool = pool.view(torch.uint8).cpu().numpy()
        got_sc = sc.cpu().numpy()
        bad = np.argwhere(got_pool != want_pool)
        assert bad.size == 0, f"{len(bad)} codes differ, first at {tuple(bad[0])}"
        assert np.array_equal(got_sc.view(np.uint32), want_sc.view(np.uint32))


@pytest.mark.parametrize("kvd", ["bf16", "i8"])
def test_prefix_sharing_with_copy_on_write(kvd):
    """A prompt written once, shared by three forks; each fork appends its
    own tokens into the partly filled shared last page (copy-on-write: the
    pool hands out a fresh page, pkv_copy_pages copies it, the new tokens go
    there), then the parent appends in place.  Every sequence decodes to the
    oracle's answer on its own logical K/V, and the prefix pages stay shared."""
    import torch

    import paged_kv_cache_266_amd as pkv
    from synth.make import _to_bits

    Hq, Hkv, D, PS, num_pages = 8, 2, 128, 16, 40
    note(f"prefix sharing: {kvd} KV, PS {PS}")
    rng = np.random.default_rng(123)
    dev = "cuda"
    byte = kvd == "i8"
    shape = (num_pages, Hkv, PS, D)
    pools = [torch.zeros(shape, dtype=torch.uint8 if byte else torch.bfloat16, device=dev) for _ in range(2)]
    if byte:
        pools = [p.view(torch.int8) for p in pools]
    scales = [torch.zeros(shape[:3], dtype=torch.float32, device=dev) for _ in range(2)] if byte else [None, None]
    host = [np.zeros(shape, dtype=np.int8 if byte else np.uint16) for _ in range(2)]
    host_sc = [np.zeros(shape[:3], dtype=np.float32) for _ in range(2)]
    def write(slots, n):
        bits = [_to_bits(rng.standard_normal((n, Hkv, D)).astype(np.float32), "bf16") for _ in range(2)]
        k_src, v_src = (torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev) for b in bits)
        pkv.write_kv(k_src, v_src, torch.from_numpy(np.asarray(slots, dtype=np.int64)).to(dev),
                     pools[0], pools[1], k_scale=scales[0], v_scale=scales[1])
        for which in range(2):
            if byte:
                exact = (bits[which].astype(np.uint32) << 16).view(np.float32)
                codes, sc = oracle.quantize_rows(exact, "i8")
                oracle.scatter_rows(host[which], np.asarray(slots), codes)
                oracle.scatter_rows(host_sc[which][..., None], np.asarray(slots), sc[..., None])
            else:
                oracle.scatter_rows(host[which], np.asarray(slots), bits[which])

    def copy(pair):
        pkv.copy_pages(torch.tensor([pair], dtype=torch.int32, device=dev), pools[0], pools[1],
                       k_scale=scales[0], v_scale=scales[1])
        for which in range(2):
            host[which][pair[1]] = host[which][pair[0]]
            host_sc[which][pair[1]] = host_sc[which][pair[0]]

    with pkv.KVPool(num_pages, PS) as pool:
        write(pool.allocate(0, 100), 100)             # 7 pages, the last holds 4 tokens
        prefix_pages = pool.pages(0)
        for child in (1, 2, 3):
            pool.fork(0, child)
        copies = []
        for child, n_new in ((1, 5), (2, 17), (3, 1)):
            with pytest.raises(pkv.SharedPage):
                pool.append_tokens(child, n_new)
            slots, pair = pool.append_tokens_cow(child, n_new)
            assert pair is not None and pair[0] == prefix_pages[-1]
            copy(pair)
            copies.append(pair)
            write(slots, n_new)
        slots, pair = pool.append_tokens_cow(0, 3)   # the parent is the page's last owner now
        assert pair is None
        write(slots, 3)
        for child in (1, 2, 3):
            assert pool.pages(child)[:6] == prefix_pages[:6]      # full prefix pages stay shared
        assert all(pool.page_owners(p) == 4 for p in prefix_pages[:6])
        ids = [0, 1, 2, 3]
        bt, ctx = pool.block_tables(ids, 8)
    torch.cuda.synchronize()
    assert list(ctx) == [103, 105, 117, 101]

    cfg = small_config(Hq, Hkv, D, "bf16", kvd, PS, tuple(int(c) for c in ctx), num_pages=num_pages)
    case = make_case(cfg, seed=5)
    written = dataclasses.replace(
        case, block_tables=bt, used_pages=np.arange(num_pages, dtype=np.int32),
        page_index=np.arange(num_pages, dtype=np.int32), k_pages=host[0], v_pages=host[1],
        k_scale=host_sc[0] if byte else None, v_scale=host_sc[1] if byte else None)
    # the device pools hold exactly the host mirror (writes and page copies)
    for which in range(2):
        got = pools[which].view(torch.int8 if byte else torch.int16).cpu().numpy()
        assert np.array_equal(got.view(host[which].dtype), host[which])
    q = upload(case, dev).q
    out = pkv.paged_attn_decode(q, pools[0], pools[1], torch.from_numpy(bt).to(dev),
                                torch.from_numpy(ctx).to(dev), case.scale,
                                max_context_len=int(ctx.max()), k_scale=scales[0], v_scale=scales[1])
    torch.cuda.synchronize()
    compare(written, out, "forked sequences")


@pytest.mark.parametrize("Hkv,D,src,kvd,PS", [
    (8, 128, "bf16", "bf16", 64),    # copy form, 16 chunks per row
    (4, 64, "f16", "f16", 16),       # copy form, 8 chunks per row
    (3, 64, "f16", "i8", 16),        # quantise, 8 lanes per row; odd head count
    (8, 128, "bf16", "fp8", 64),     # quantise, 16 lanes per row
])
def test_append_many_rows_skips_out_of_range_slots(Hkv, D, src, kvd, PS):
    """Thousands of rows (several grid passes and a ragged last block) with
    slots -1 and num_pages * page_size among them: those rows are skipped,
    every other row lands at its slot (bit for bit against the oracle's
    quantiser and scatter), and nothing else in the pools changes."""
    import torch

    import paged_kv_cache_266_amd as pkv
    from synth.make import _to_bits

    note(f"append many rows: Hkv {Hkv} D {D} {src}->{kvd} PS {PS}")
    rng = np.random.default_rng(4242)
    n, num_pages = 3001, 256
    slots = rng.permutation(num_pages * PS)[:n].astype(np.int64)
    slots[7] = -1
    slots[1000] = num_pages * PS
    valid = (slots >= 0) & (slots < num_pages * PS)
    dev = "cuda"
    shape = (num_pages, Hkv, PS, D)
    byte = kvd in ("i8", "fp8")
    kv_t = torch_dtype(kvd)
    fill = 0x5A
    pools = [torch.full(shape, fill, dtype=torch.uint8, device=dev) for _ in range(2)]
    if not byte:
        pools = [torch.full((*shape[:3], 2 * D), fill, dtype=torch.uint8, device=dev) for _ in range(2)]
    pools = [p.view(kv_t) for p in pools]
    scales = [torch.full(shape[:3], -7.0, dtype=torch.float32, device=dev) for _ in range(2)] if byte else [None, None]
    want = []
    new = []
    for _ in range(2):
        x = rng.standard_normal((n, Hkv, D)).astype(np.float32)
        bits = _to_bits(x, src)
        new.append(_as_torch(bits, src, dev))
        row_bytes = D * (1 if byte else 2)
        want_pool = np.full((*shape[:3], row_bytes), fill, dtype=np.uint8)
        want_sc = np.full(shape[:3], -7.0, dtype=np.float32)
        if byte:
            exact = (bits.view(np.float16).astype(np.float32) if src == "f16"
                     else (bits.astype(np.uint32) << 16).view(np.float32))
            codes, s = oracle.quantize_rows(exact[valid], kvd)
            oracle.scatter_rows(want_pool, slots[valid], codes.view(np.uint8))
            oracle.scatter_rows(want_sc[..., None], slots[valid], s[..., None])
        else:
            oracle.scatter_rows(want_pool, slots[valid], bits[valid].view(np.uint8).reshape(-1, Hkv, row_bytes))
        want.append((want_pool, want_sc))
    pkv.write_kv(new[0], new[1], torch.from_numpy(slots).to(dev), pools[0], pools[1],
                 k_scale=scales[0], v_scale=scales[1])
    torch.cuda.synchronize()
    for w, (want_pool, want_sc) in enumerate(want):
        got = pools[w].view(torch.uint8).cpu().numpy().reshape(want_pool.shape)
        bad = np.argwhere(got != want_pool)
        assert bad.size == 0, f"pool {w}: {len(bad)} bytes differ, first at {tuple(bad[0])}"
        if byte:
            assert np.array_equal(scales[w].cpu().numpy().view(np.uint32), want_sc.view(np.uint32))


@pytest.mark.parametrize("Hkv,D,kvd,PS", [
    (2, 64, "f16", 16),      # 4 KiB pages: one partial tile
    (8, 128, "bf16", 64),    # 128 KiB pages: eight tiles
    (3, 128, "i8", 16),      # 6 KiB pages with scales
    (8, 128, "fp8", 64),     # 64 KiB pages with scales
])
def test_copy_pages_whole_pages(Hkv, D, kvd, PS):
    """pkv_copy_pages copies whole pages (codes and scales, K and V) onto
    their destinations; a pair naming a page outside the pool is skipped and
    every other page is untouched."""
    import torch

    import paged_kv_cache_266_amd as pkv

    note(f"copy pages: Hkv {Hkv} D {D} {kvd} PS {PS}")
    rng = np.random.default_rng(99)
    num_pages = 300
    byte = kvd in ("i8", "fp8")
    e = 1 if byte else 2
    dev = "cuda"
    host = [rng.integers(0, 256, size=(num_pages, Hkv, PS, D * e), dtype=np.uint8) for _ in range(2)]
    if byte and kvd == "fp8":
        for h in host:
            h[(h & 0x7F) == 0x7F] = 0x10      # no NaN codes
    host_sc = [rng.standard_normal((num_pages, Hkv, PS)).astype(np.float32) for _ in range(2)]
    pools = [torch.from_numpy(h).to(dev).view(torch_dtype(kvd)).view(num_pages, Hkv, PS, D) for h in host]
    scales = [torch.from_numpy(h).to(dev) for h in host_sc] if byte else [None, None]
    perm = rng.permutation(num_pages)
    src, dst = perm[:100], perm[100:200]
    pairs = np.stack([src, dst], 1).astype(np.int32)
    pairs[5] = (-1, pairs[5, 1])             # skipped
    pairs[6] = (pairs[6, 0], num_pages)      # skipped
    pkv.copy_pages(torch.from_numpy(pairs).to(dev), pools[0], pools[1], k_scale=scales[0], v_scale=scales[1])
    torch.cuda.synchronize()
    for w in range(2):
        want = host[w].copy()
        want_sc = host_sc[w].copy()
        for s_, d_ in pairs:
            if 0 <= s_ < num_pages and 0 <= d_ < num_pages:
                want[d_] = host[w][s_]
                want_sc[d_] = host_sc[w][s_]
        got = pools[w].view(torch.uint8).cpu().numpy().reshape(want.shape)
        assert np.array_equal(got, want)
        if byte:
            assert np.array_equal(scales[w].cpu().numpy().view(np.uint32), want_sc.view(np.uint32))
