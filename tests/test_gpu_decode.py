"""GPU parity of the HIP decode path with the fp64 oracle (needs a gfx950 GPU).

Every test calls the C ABI (through the thin Python binding) on seeded
synthetic inputs and compares element by element with the oracle, within the
max-abs tolerances 4e-3 (f16 KV), 1.6e-2 (bf16 KV), 2.5e-2 (int8 KV).
"""

import itertools

import numpy as np
import pytest

import oracle
from gpu_helpers import TOL, compare, gpu_decode, note, small_config, to_f64
from synth import CONFIGS, make_case
from synth.configs import ORDER
from synth.device import upload
from synth.make import repermute

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_266_amd as pkv

    pkv.lib()  # fail loudly if the library is missing
    yield


# ---------------------------------------------------------------------------
# The five workloads at full size, in the launch configuration the benchmark
# times (default partition length), compared on every output element.

@pytest.mark.parametrize("name", ORDER + ["llama3_8b_gqa_fp8"])
def test_parity_full_config(name):
    cfg = CONFIGS[name]
    note(f"[parity] {name}: B={cfg.batch} Hq={cfg.num_q_heads} Hkv={cfg.num_kv_heads} "
         f"D={cfg.head_dim} PS={cfg.page_size} kv={cfg.kv_dtype} seed={cfg.seed}")
    case = make_case(cfg)
    out = gpu_decode(case)
    compare(case, out, name)


# ---------------------------------------------------------------------------
# Every compiled instantiation on small ragged batches that span several
# 64-token tiles and a partial last page, with the batch's tiles split over
# the default grid, over 3 waves (segments cut across waves) and over 40
# waves (about one tile each, many pieces per segment).

SUPPORTED = [(D, PS, G, qd, kvd)
             for D, PS, G in itertools.product((64, 128), (16, 64), (1, 2, 4, 8))
             for qd, kvd in (("f16", "f16"), ("bf16", "bf16"), ("f16", "i8"), ("bf16", "i8"),
                             ("f16", "fp8"), ("bf16", "fp8"))]


@pytest.mark.parametrize("D,PS,G,qd,kvd", SUPPORTED)
def test_parity_every_instantiation(D, PS, G, qd, kvd):
    lens = (1, 63, 64, 65, 300, 777)
    Hkv = 2
    cfg = small_config(G * Hkv, Hkv, D, qd, kvd, PS, lens)
    note(f"[inst] D={D} PS={PS} G={G} q={qd} kv={kvd} lens={lens}")
    case = make_case(cfg, seed=100 + D + PS + G)
    for splits in (0, 3, 40):
        out = gpu_decode(case, num_splits=splits)
        compare(case, out, f"splits={splits}")


def test_edge_lengths():
    ps = 64
    lens = (0, 1, ps - 1, ps, ps + 1, 511, 512, 513, 1023, 1024, 1025, 2048)
    cfg = small_config(32, 8, 128, "bf16", "bf16", ps, lens)
    note(f"[edge] lens={lens}")
    case = make_case(cfg, seed=7)
    out = gpu_decode(case)
    g = to_f64(out)
    assert (g[0] == 0).all(), "empty sequence must give zeros"
    compare(case, out, "edge")


def test_poisoned_tails_do_not_leak():
    """NaN in every unused slot of used pages and in every unused page."""
    for name in ("tiny", "qwen_1p8b_int8"):
        cfg = CONFIGS[name]
        note(f"[poison] {name}")
        clean = make_case(cfg)
        poisoned = make_case(cfg, poison=True)
        a = gpu_decode(clean)
        b = gpu_decode(poisoned)
        assert np.isfinite(to_f64(b)).all()
        assert torch_equal_bits(a.cpu(), b.cpu())
        compare(poisoned, b, name + " poisoned")


@pytest.mark.parametrize("Hq,Hkv,qd,PS", [(32, 8, "bf16", 64), (16, 16, "f16", 16), (8, 1, "bf16", 16)])
def test_poisoned_tails_do_not_leak_fp8(Hq, Hkv, qd, PS):
    """E4M3 NaN codes (and NaN scales) in every slot past each sequence's
    end: the output is finite and bitwise equal to the clean cache's."""
    lens = (1, 15, 16, 17, 63, 64, 65, 200, 1000)
    cfg = small_config(Hq, Hkv, 128, qd, "fp8", PS, lens)
    note(f"[poison fp8] Hq={Hq} Hkv={Hkv} q={qd} PS={PS}")
    clean = make_case(cfg, seed=31)
    poisoned = make_case(cfg, seed=31, poison=True)
    a = gpu_decode(clean)
    b = gpu_decode(poisoned)
    assert np.isfinite(to_f64(b)).all()
    assert torch_equal_bits(a.cpu(), b.cpu())
    compare(poisoned, b, "fp8 poisoned")


@pytest.mark.parametrize("qd,kvd,PS", [("bf16", "bf16", 16), ("bf16", "bf16", 64), ("f16", "i8", 16),
                                       ("bf16", "fp8", 16), ("f16", "fp8", 64)])
def test_out_of_pool_block_table_entry_gives_nan_for_that_sequence_only(qd, kvd, PS):
    """A block-table entry the sequence needs that lies outside the pool
    (in its first tile, or in a middle one) makes that sequence's output NaN
    -- every head, since all KV heads read the page -- and leaves every other
    sequence equal to the oracle, however the tiles are split over waves
    (a bad first tile right after another segment in the same wave's range
    included)."""
    import dataclasses

    lens = (200, 130, 64, 300, 90)
    cfg = small_config(32, 8, 128, qd, kvd, PS, lens)
    note(f"[out-of-pool] q={qd} kv={kvd} PS={PS}")
    clean = make_case(cfg, seed=55)
    bt = clean.block_tables.copy()
    bt[1, 0] = cfg.num_pages + 5            # first tile of sequence 1
    bt[3, (128 + 10) // PS] = -7            # a middle tile of sequence 3
    bad = dataclasses.replace(clean, block_tables=bt)
    ref = oracle.paged_decode(clean)
    good = [0, 2, 4]
    from gpu_helpers import TOL
    for splits in (0, 1, 2, 3, 7, 40):
        g = to_f64(gpu_decode(bad, num_splits=splits))
        assert np.isnan(g[1]).all() and np.isnan(g[3]).all(), splits
        assert np.isfinite(g[good]).all(), splits
        assert np.abs(g[good] - ref[good]).max() <= TOL[kvd], splits


@pytest.mark.parametrize("kvd,qd", [("bf16", "bf16"), ("fp8", "bf16")])
def test_one_million_token_context(kvd, qd):
    """One sequence of 2^20 tokens (8x the 128k workload) spread over the
    whole grid and merged, next to a 1-token sequence."""
    n = 1 << 20
    cfg = small_config(8, 1, 128, qd, kvd, 64, (n, 1), num_pages=(n // 64) + 8)
    note(f"[max context] {n} tokens, kv={kvd}")
    case = make_case(cfg, seed=77)
    out = gpu_decode(case)
    compare(case, out, "1M tokens")


def test_four_thousand_sequences():
    """A batch of 4096 short ragged sequences (lengths 0..130): more segments
    than waves, many empty ones, every wave crossing many segment ends."""
    rng = np.random.default_rng(8)
    lens = tuple(int(x) for x in rng.integers(0, 131, size=4096))
    cfg = small_config(8, 2, 64, "f16", "f16", 16, lens)
    note("[max batch] 4096 sequences")
    case = make_case(cfg, seed=9)
    for splits in (0, 1024, 5000):
        out = gpu_decode(case, num_splits=splits)
        compare(case, out, f"4096 seqs, splits={splits}")
        g = to_f64(out)
        assert (g[np.asarray(lens) == 0] == 0).all()


def test_page_permutation_invariance_bitwise():
    cfg = CONFIGS["llama3_8b_gqa"]
    note("[perm] llama3_8b_gqa, 2 re-permutations")
    case = make_case(cfg)
    base = gpu_decode(case).cpu()
    for s in (1, 2):
        moved = repermute(case, seed=s)
        got = gpu_decode(moved).cpu()
        assert torch_equal_bits(base, got)


def test_run_to_run_determinism_bitwise():
    cfg = CONFIGS["long_128k"]
    note("[determinism] long_128k x3")
    case = make_case(cfg)
    dev = upload(case, "cuda")
    outs = [gpu_decode(case, dev=dev).cpu() for _ in range(3)]
    assert torch_equal_bits(outs[0], outs[1]) and torch_equal_bits(outs[0], outs[2])


def test_split_and_unsplit_agree():
    cfg = small_config(32, 8, 128, "bf16", "bf16", 64, (4096, 3000, 777, 64))
    note("[split] 1 / 7 / 64 / 2000 waves and the default")
    case = make_case(cfg, seed=21)
    dev = upload(case, "cuda")
    outs = {n: to_f64(gpu_decode(case, num_splits=n, dev=dev)) for n in (1, 7, 64, 2000, 0)}
    for n, o in outs.items():
        assert np.abs(o - outs[1]).max() <= 1.6e-2, n
        compare(case, gpu_decode(case, num_splits=n, dev=dev), f"splits={n}")


def test_gqa_equals_mha_with_repeated_kv():
    cfg = small_config(8, 2, 128, "bf16", "bf16", 64, (300, 1000))
    note("[gqa] G=4 vs repeated-KV G=1")
    case = make_case(cfg, seed=4)
    mha = make_case(cfg, seed=4)
    fields = {k: v for k, v in cfg.__dict__.items() if k != "name"}
    fields["num_kv_heads"] = 8
    from synth import get_config

    mha.cfg = get_config("tiny", **fields)
    mha.k_pages = np.repeat(case.k_pages, 4, axis=1)
    mha.v_pages = np.repeat(case.v_pages, 4, axis=1)
    ga, gb = gpu_decode(case), gpu_decode(mha)
    compare(case, ga, "G=4")
    compare(mha, gb, "repeated KV, G=1")
    assert np.allclose(oracle.paged_decode(case), oracle.paged_decode(mha), rtol=0, atol=1e-12)
    assert np.abs(to_f64(ga) - to_f64(gb)).max() <= 1.6e-2


def _two_launch(case, dev, num_splits=0):
    """The unfused form: partition kernel, then merge kernel, same workspace."""
    import ctypes

    import torch

    import paged_kv_cache_266_amd as pkv
    from paged_kv_cache_266_amd._lib import check, lib

    cfg = case.cfg
    out = torch.empty_like(dev.q)
    a = pkv.decode_args(dev.q, dev.k_pool, dev.v_pool, dev.block_tables, dev.context_lens, case.scale,
                        max_context_len=cfg.max_context_len, out=out, k_scale=dev.k_scale,
                        v_scale=dev.v_scale, num_splits=num_splits)
    ws = pkv.alloc_workspace(a, dev.q.device)
    a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()   # no merge counters needed
    sh = torch.cuda.current_stream().cuda_stream
    check(lib().pkv_paged_attn_decode_partitions(ctypes.byref(a), sh))
    check(lib().pkv_splitk_reduce(ctypes.byref(a), sh))
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("lens,splits,kvd", [
    ((4096, 3000, 777, 64, 0, 1), 0, "bf16"),        # ragged GQA batch, default grid
    ((65536,), 1000, "bf16"),                        # one segment shared by 1000 waves: 4 merge levels
    ((20000, 9, 20000), 300, "bf16"),
    ((20000, 9, 20000), 2000, "bf16"),               # more waves than SIMDs: weighted shares
    ((20000, 9, 20000), 1500, "fp8"),                # the same on the matrix-core kernel
])
def test_one_launch_and_two_launch_forms_agree(lens, splits, kvd):
    cfg = small_config(32, 8, 128, "bf16", kvd, 64, lens)
    note(f"[fused vs two-launch] lens {lens} splits {splits} kv {kvd}")
    case = make_case(cfg, seed=31)
    dev = upload(case, "cuda")
    one = gpu_decode(case, num_splits=splits, dev=dev)
    two = _two_launch(case, dev, num_splits=splits)
    compare(case, one, "one launch")
    compare(case, two, "two launches")
    assert np.abs(to_f64(one) - to_f64(two)).max() <= TOL[kvd]


def test_buffers_reused_across_shapes_and_counters_return_to_zero():
    """One workspace and one merge-counter array serve calls of different
    shapes in turn; after each, every counter is zero again and every output
    is right."""
    import ctypes

    import torch

    import paged_kv_cache_266_amd as pkv
    from paged_kv_cache_266_amd._lib import check, lib

    note("[buffer reuse] big, small, big, small")
    big = make_case(small_config(32, 8, 128, "bf16", "bf16", 64, (30000, 5000, 64, 4000)), seed=41)
    small = make_case(small_config(32, 8, 128, "bf16", "bf16", 64, (700, 65)), seed=42)
    cases = [big, small, big, small]
    devs = {id(c): upload(c, "cuda") for c in (big, small)}
    args = []
    for c in cases:
        d = devs[id(c)]
        out = torch.empty_like(d.q)
        a = pkv.decode_args(d.q, d.k_pool, d.v_pool, d.block_tables, d.context_lens, c.scale,
                            max_context_len=c.cfg.max_context_len, out=out, num_splits=600)
        args.append((c, a, out))
    ws = pkv.alloc_workspace(args[0][1], "cuda")          # the bigger of the two shapes
    ws.fill_(0xA5)                                        # contents between calls do not matter
    ctr = pkv.alloc_merge_counters(args[0][1], "cuda")
    for c, a, out in args:
        a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
        a.merge_counters, a.merge_counter_bytes = ctr.data_ptr(), 4 * ctr.numel()
        check(lib().pkv_paged_attn_decode(ctypes.byref(a), torch.cuda.current_stream().cuda_stream))
        torch.cuda.synchronize()
        compare(c, out, f"B={c.cfg.batch}")
        assert int(ctr.abs().sum()) == 0


def torch_equal_bits(a, b):
    import torch

    return bool(torch.equal(a.view(torch.int16), b.view(torch.int16)))


@pytest.mark.parametrize("n,PS,kvd", [(1048576, 64, "bf16"), (393217, 16, "i8"), (524288, 64, "fp8")])
def test_contexts_far_beyond_128k(n, PS, kvd):
    """One sequence of up to a million tokens (contexts beyond 128k, GQA 32/8)
    beside short ones, default wave count: every output against the oracle
    (token, tile and block-table indices far past 2^16, pools over 2 GiB)."""
    lens = (n, 3, 1000)
    cfg = small_config(32, 8, 128, "bf16", kvd, PS, lens, num_pages=sum(-(-x // PS) for x in lens) + 40)
    note(f"[long context] n={n} PS={PS} kv={kvd}")
    case = make_case(cfg, seed=777)
    compare(case, gpu_decode(case), f"{n} tokens")
