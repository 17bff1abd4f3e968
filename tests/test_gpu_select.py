"""GPU parity of lcs_select_topk.

* Bit-exact: the CPU rule in the pinned fp32 order, run on the GPU's own logits,
  gives identical index arrays and counts.
* Against oracle logits: at least 99% overlap with the fp64 selection (near-ties
  at the k-th place may legitimately swap between fp32 and fp64 scores).
"""
import numpy as np
import pytest

from long_context_self_amd import synth
from oracle import attention as oa
from oracle import select as osel

from gpu_helpers import bf16_dev, i32_dev, kv_dev, require_gpu, scale_for

pytestmark = pytest.mark.gpu


def gpu_select(logits_np, prefix_len, Hkv, mode, top_k, n_sink, n_recent, bs=0, poison=True):
    torch, lcs = require_gpu()
    lg = torch.from_numpy(np.ascontiguousarray(logits_np, dtype=np.float32)).cuda()
    pl = i32_dev(prefix_len, torch)
    idx, cnt = lcs.select_topk(lg, pl, int(np.max(prefix_len)), Hkv, mode, top_k, n_sink, n_recent,
                               block_size=bs)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), cnt.cpu().numpy()


def cpu_rule(logits_np, prefix_len, Hkv, mode, top_k, n_sink, n_recent, bs=0, precision="f32"):
    res = osel.select(logits_np, prefix_len, Hkv, mode, top_k, n_sink, n_recent, bs, precision)
    return res


def assert_exact(idx, cnt, res):
    for b in range(len(res)):
        for s in range(len(res[b])):
            ref = res[b][s]
            assert cnt[b, s] == ref.size, f"count b={b} s={s}: {cnt[b, s]} vs {ref.size}"
            assert np.array_equal(idx[b, s, :ref.size], ref), f"indices differ at b={b} s={s}"


def gpu_logits(cfg, kv, q):
    torch, lcs = require_gpu()
    dkv = kv_dev(kv, torch, lcs)
    maxL = int(kv.prefix_len.max())
    _, logits, _ = lcs.verify_attn(dkv, bf16_dev(q, torch), i32_dev(kv.prefix_len, torch), maxL,
                                   scale_for(cfg.d), (0, q.shape[1] - 1))
    torch.cuda.synchronize()
    return logits.cpu().numpy()


@pytest.mark.parametrize("name,L,B,mode", [("tiny", None, 1, "shared"),
                                           ("llama8b_32k", 8192, 1, "shared"),
                                           ("qwen14b_64k", 9000, 2, "per_kv_head"),
                                           ("stress_128k", 5000, 3, "shared")])
def test_bit_exact_on_gpu_logits_and_overlap(name, L, B, mode):
    cfg = synth.CONFIGS[name]
    cfg = cfg.with_(B=B, L=L if L else cfg.L)
    lens = [cfg.L - 101 * b for b in range(B)]
    top_k = min(cfg.top_k, cfg.L // 8)
    kv = synth.make_paged_kv(cfg, seed=7, lens=lens)
    q = synth.make_queries(cfg, kv, cfg.n_q, seed=7)
    glog = gpu_logits(cfg, kv, q)
    idx, cnt = gpu_select(glog, kv.prefix_len, cfg.Hkv, mode, top_k, cfg.n_sink, cfg.n_recent)
    assert_exact(idx, cnt, cpu_rule(glog, kv.prefix_len, cfg.Hkv, mode, top_k, cfg.n_sink, cfg.n_recent))
    # against the fp64 oracle end to end
    _, olog, _ = oa.verify_attn(q, kv.k, kv.v, kv.block_table, kv.prefix_len, cfg.page_size,
                                scale_for(cfg.d))
    ref = osel.select(olog, kv.prefix_len, cfg.Hkv, mode, top_k, cfg.n_sink, cfg.n_recent)
    for b in range(B):
        for s in range(len(ref[b])):
            got = set(idx[b, s, :cnt[b, s]].tolist())
            overlap = len(got & set(ref[b][s].tolist())) / ref[b][s].size
            assert overlap >= 0.99, f"overlap {overlap}"


@pytest.mark.parametrize("mode", ["shared", "per_kv_head", "block"])
def test_ties_and_ragged(mode):
    rng = np.random.default_rng(3)
    B, Hq, Hkv = 3, 8, 2
    lens = np.array([9000, 4096, 777], dtype=np.int32)
    ld = 9004
    lg = (rng.integers(-3, 4, size=(B, Hq, 2, ld))).astype(np.float32)   # heavy ties
    lg[:, :, :, 100] = -0.0
    bs = 16 if mode == "block" else 0
    k = 40 if mode == "block" else 600
    idx, cnt = gpu_select(lg, lens, Hkv, mode, k, 5, 33, bs)
    assert_exact(idx, cnt, cpu_rule(lg, lens, Hkv, mode, k, 5, 33, bs))


@pytest.mark.parametrize("mode", ["shared", "per_kv_head", "block"])
def test_one_bin_holds_every_candidate(mode):
    """All scores equal: the whole pool lands in one first-digit bin, more candidates
    than a workgroup holds in LDS, and ties go to the smaller index."""
    lens = np.array([60000, 33333], dtype=np.int32)
    lg = np.full((2, 4, 2, 60000), 0.75, dtype=np.float32)
    bs = 16 if mode == "block" else 0
    k = 300 if mode == "block" else 5000
    idx, cnt = gpu_select(lg, lens, 2, mode, k, 4, 64, bs)
    assert_exact(idx, cnt, cpu_rule(lg, lens, 2, mode, k, 4, 64, bs))


@pytest.mark.parametrize("mode", ["shared", "per_kv_head"])
def test_sets_around_64k_items(mode):
    """Sets just above and at 2^16 items (many 4096-item chunks, a ragged last chunk)
    give the CPU rule's result."""
    rng = np.random.default_rng(6)
    lens = np.array([70001, 65536, 1000], dtype=np.int32)
    lg = rng.standard_normal((3, 4, 2, 70004)).astype(np.float32)
    idx, cnt = gpu_select(lg, lens, 2, mode, 3000, 4, 64)
    assert_exact(idx, cnt, cpu_rule(lg, lens, 2, mode, 3000, 4, 64))
    idx2, cnt2 = gpu_select(lg[1:, :, :, :65536].copy(), lens[1:], 2, mode, 3000, 4, 64)
    assert_exact(idx2, cnt2, cpu_rule(lg[1:, :, :, :65536], lens[1:], 2, mode, 3000, 4, 64))


@pytest.mark.parametrize("mode", ["shared", "block"])
def test_short_context_keeps_everything(mode):
    rng = np.random.default_rng(4)
    lens = np.array([50, 0, 3], dtype=np.int32)
    lg = rng.standard_normal((3, 4, 2, 64)).astype(np.float32)
    bs = 8 if mode == "block" else 0
    idx, cnt = gpu_select(lg, lens, 2, mode, 64, 4, 16, bs)
    assert_exact(idx, cnt, cpu_rule(lg, lens, 2, mode, 64, 4, 16, bs))


def test_zero_k_and_windows_only():
    rng = np.random.default_rng(5)
    lens = np.array([5000], dtype=np.int32)
    lg = rng.standard_normal((1, 4, 2, 5000)).astype(np.float32)
    idx, cnt = gpu_select(lg, lens, 2, "shared", 0, 4, 64)
    assert_exact(idx, cnt, cpu_rule(lg, lens, 2, "shared", 0, 4, 64))


def test_deterministic_repeat():
    rng = np.random.default_rng(6)
    lens = np.array([40000, 39000], dtype=np.int32)
    lg = rng.standard_normal((2, 8, 2, 40000)).astype(np.float32)
    a = gpu_select(lg, lens, 8, "per_kv_head", 2048, 4, 64)
    b = gpu_select(lg, lens, 8, "per_kv_head", 2048, 4, 64)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert_exact(a[0], a[1], cpu_rule(lg, lens, 8, "per_kv_head", 2048, 4, 64))


def test_full_stress_128k_shape():
    """Full 128K x B8 shape of the long-context workload on synthetic logits."""
    rng = np.random.default_rng(8)
    cfg = synth.CONFIGS["stress_128k"]
    lens = np.full(cfg.B, cfg.L, dtype=np.int32)
    lg = (rng.standard_normal((cfg.B, cfg.Hq, 2, cfg.L)) * 1.4).astype(np.float32)
    idx, cnt = gpu_select(lg, lens, cfg.Hkv, "shared", cfg.top_k, cfg.n_sink, cfg.n_recent)
    for b in (0, cfg.B - 1):        # CPU rule on two of the eight sequences
        ref = osel.topk_tokens(osel.scores_f32_pinned(lg, b, cfg.L, range(cfg.Hq)), cfg.L,
                               cfg.top_k, cfg.n_sink, cfg.n_recent)
        assert cnt[b, 0] == ref.size and np.array_equal(idx[b, 0, :ref.size], ref)


@pytest.mark.parametrize("maxlen", [262144, 262160, 300001])
def test_sets_at_and_beyond_one_workgroup(maxlen):
    """Sets of 2^18 items and just above (64 and 65 chunks of 4096 items, a ragged last
    chunk), with random scores and with every pool item in one first-digit bin (far more
    candidates than LDS holds), give the CPU rule's result."""
    rng = np.random.default_rng(9)
    lens = np.array([maxlen, maxlen - 4097], dtype=np.int32)
    lg = rng.standard_normal((2, 2, 2, maxlen)).astype(np.float32)
    idx, cnt = gpu_select(lg, lens, 1, "shared", 9000, 4, 64)
    assert_exact(idx, cnt, cpu_rule(lg, lens, 1, "shared", 9000, 4, 64))
    flat = np.full((2, 2, 2, maxlen), -0.5, dtype=np.float32)
    idx, cnt = gpu_select(flat, lens, 1, "shared", 9000, 4, 64)
    assert_exact(idx, cnt, cpu_rule(flat, lens, 1, "shared", 9000, 4, 64))


def test_full_llama8b_32k_shape():
    """The Llama-3-8B-shaped workload at its full size (32K, 32 query heads, top-2048 + 4
    sink + 64 recent): bit-exact against the pinned-order CPU rule on the GPU's own
    logits, and at least 99 % overlap with the selection the fp64 oracle makes from its
    own logits."""
    cfg = synth.CONFIGS["llama8b_32k"]
    kv = synth.make_paged_kv(cfg, seed=0)
    q = synth.make_queries(cfg, kv, cfg.n_q, seed=0)
    glog = gpu_logits(cfg, kv, q)
    idx, cnt = gpu_select(glog, kv.prefix_len, cfg.Hkv, "shared", cfg.top_k, cfg.n_sink, cfg.n_recent)
    assert_exact(idx, cnt, cpu_rule(glog, kv.prefix_len, cfg.Hkv, "shared", cfg.top_k, cfg.n_sink,
                                     cfg.n_recent))
    _, olog, _ = oa.verify_attn(q, kv.k, kv.v, kv.block_table, kv.prefix_len, cfg.page_size,
                                scale_for(cfg.d))
    ref = osel.select(olog, kv.prefix_len, cfg.Hkv, "shared", cfg.top_k, cfg.n_sink, cfg.n_recent)[0][0]
    got = set(idx[0, 0, :cnt[0, 0]].tolist())
    overlap = len(got & set(ref.tolist())) / ref.size
    assert cnt[0, 0] == ref.size == cfg.n_sink + cfg.top_k + cfg.n_recent
    assert overlap >= 0.99, f"overlap {overlap}"


def test_largest_accepted_set():
    """max_prefix_len = 2^24 - 1, the largest the ABI accepts: item indices fill the 24
    bits of the composites and the grid spans all 4096 chunks.  Bit-exact against the CPU
    rule on the same scores."""
    L = (1 << 24) - 1
    rng = np.random.default_rng(10)
    lg = rng.standard_normal((1, 1, 2, L), dtype=np.float32)
    lens = np.array([L], dtype=np.int32)
    idx, cnt = gpu_select(lg, lens, 1, "shared", 5000, 4, 64)
    assert_exact(idx, cnt, cpu_rule(lg, lens, 1, "shared", 5000, 4, 64))
    assert idx[0, 0, cnt[0, 0] - 1] == L - 1


@pytest.mark.parametrize("mode,bs", [("shared", 0), ("per_kv_head", 0), ("block", 16)])
@pytest.mark.parametrize("which", ["top_k", "n_sink", "n_recent"])
def test_window_sizes_at_int32_max_keep_everything(mode, bs, which):
    """top_k, n_sink or n_recent at INT32_MAX: the budget covers every item, so every
    position (or block) is kept, as the CPU rule says; the device's 32-bit window sums
    must not overflow into a partial selection."""
    rng = np.random.default_rng(31)
    B, Hq, Hkv, ld = 2, 4, 2, 700
    lens = np.array([700, 333], dtype=np.int32)
    lg = rng.standard_normal((B, Hq, 2, ld)).astype(np.float32)
    sizes = {"top_k": 5, "n_sink": 2, "n_recent": 3}
    sizes[which] = 2 ** 31 - 1
    idx, cnt = gpu_select(lg, lens, Hkv, mode, sizes["top_k"], sizes["n_sink"], sizes["n_recent"], bs=bs)
    res = cpu_rule(lg, lens, Hkv, mode, sizes["top_k"], sizes["n_sink"], sizes["n_recent"], bs=bs)
    for b in range(B):
        n_items = -(-int(lens[b]) // bs) if mode == "block" else int(lens[b])
        for s in range(len(res[b])):
            assert res[b][s].tolist() == list(range(n_items))
    assert_exact(idx, cnt, res)


@pytest.mark.parametrize("mode,bs", [("shared", 0), ("per_kv_head", 0), ("block", 64)])
def test_workspace_reuse_garbage_and_layout_changes(mode, bs):
    """One workspace through a sequence of calls: first filled with random bytes (the
    histograms are then rebuilt from the keys), then reused with the same layout (the
    histograms the last call left clean are trusted), then with another layout and back.
    Every call equals the CPU rule bit for bit."""
    torch, lcs = require_gpu()
    rng = np.random.default_rng(21)
    Hq, Hkv = 8, 2
    shapes = [(2, 9000), (2, 9000), (3, 5000), (2, 9000)]
    need = max(lcs.select_workspace_bytes(B, Hq, Hkv, mode, L, bs) for B, L in shapes)
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    ws = torch.randint(0, 256, (need,), dtype=torch.uint8, device="cuda", generator=g)
    for B, L in shapes:
        lens = np.array([L - 37 * b for b in range(B)], dtype=np.int32)
        lg_np = rng.standard_normal((B, Hq, 2, L)).astype(np.float32)
        lg = torch.from_numpy(lg_np).cuda()
        top_k = 40 if mode == "block" else 700
        idx, cnt = lcs.select_topk(lg, i32_dev(lens, torch), L, Hkv, mode, top_k, 4, 64, block_size=bs,
                                   workspace=ws)
        torch.cuda.synchronize()
        assert_exact(idx.cpu().numpy(), cnt.cpu().numpy(), cpu_rule(lg_np, lens, Hkv, mode, top_k, 4, 64, bs))


def _boundary_bin_logits(rng, B, L, Hq, n_c, n_high, n_sink, n_recent):
    """Logits whose set scores put n_high items above one first-digit bin and exactly
    n_c tied items in it (every head's two rows hold the same value v, so every score
    is the same sum of v), the rest below it."""
    lens = np.array([L - 37 * b for b in range(B)], dtype=np.int32)
    v = np.full((B, L), 0.001, dtype=np.float32)
    for b in range(B):
        pool = rng.permutation(np.arange(n_sink, lens[b] - n_recent))
        assert pool.size > n_high + n_c
        v[b, pool[:n_high]] = (100.0 + rng.random(n_high)).astype(np.float32)
        v[b, pool[n_high:n_high + n_c]] = 1.0
    lg = np.ascontiguousarray(np.broadcast_to(v[:, None, None, :], (B, Hq, 2, L)), dtype=np.float32)
    return lg, lens


@pytest.mark.parametrize("mode", ["shared", "per_kv_head"])
@pytest.mark.parametrize("n_c", [1023, 1024, 1025, 3000, 8192, 8193])
def test_boundary_bin_sizes_around_prefetch_and_lds(mode, n_c):
    """The boundary bin holds exactly n_c tied items: around the 1024 candidates the
    finish pass loads before it knows their count, and around the 8192 it holds in LDS
    (one more are read from memory in every radix pass).  200 of them are kept, the
    smaller indices first, as the CPU rule keeps them (finish with 1024 threads)."""
    rng = np.random.default_rng(100 + n_c)
    K, n_high = 2048, 1848
    lg, lens = _boundary_bin_logits(rng, 1, 40000, 4, n_c, n_high, 4, 64)
    idx, cnt = gpu_select(lg, lens, 2, mode, K, 4, 64)
    assert_exact(idx, cnt, cpu_rule(lg, lens, 2, mode, K, 4, 64))


@pytest.mark.parametrize("B", [3, 7])
@pytest.mark.parametrize("n_c", [1025, 8193])
def test_boundary_bin_sizes_smaller_finish_workgroups(B, n_c):
    """The same at 360000-item sets (88 chunks each): over three sequences the finish pass
    runs 512-thread workgroups (264 of them, two per CU; two prefetched candidates per
    thread), over seven 256-thread ones (616; four per thread)."""
    rng = np.random.default_rng(200 + n_c + B)
    K, n_high = 2048, 1848
    lg, lens = _boundary_bin_logits(rng, B, 360000, 4, n_c, n_high, 4, 64)
    idx, cnt = gpu_select(lg, lens, 2, "shared", K, 4, 64)
    assert_exact(idx, cnt, cpu_rule(lg, lens, 2, "shared", K, 4, 64))
