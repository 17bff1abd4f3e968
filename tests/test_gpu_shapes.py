"""GPU parity over the shapes the ABI accepts beyond the five workloads: page sizes below
the 16-token MFMA tile (1, 2, 4, 8) and above it (128, 256, and the largest, 1024), one
query head per KV head (G = 1) up to the largest, 64, a single verifier row (n_q = 1),
head dim 64 in every call, prefixes of one token, and row sets split over two or three
48-row chunks.  Each case runs verify, select and single-token draft steps against the
fp64 oracle, with the tolerances of the other GPU tests (outputs 1e-2 max-abs, logits
1e-3 relative, selection bit-exact against the pinned-order CPU rule on the GPU's own
logits)."""
import numpy as np
import pytest

from long_context_self_amd import synth

from gpu_helpers import require_gpu
from test_gpu_select import assert_exact, cpu_rule, gpu_select
from test_gpu_sparse import check as sparse_check
from test_gpu_sparse import selected
from test_gpu_verify import check as verify_check
from test_gpu_verify import run_verify

pytestmark = pytest.mark.gpu

# (page_size, Hq, Hkv, d, n_q, prefix lengths)
CASES = [
    (1, 8, 2, 128, 3, [300, 257]),
    (2, 8, 1, 64, 7, [333, 64]),
    (4, 16, 1, 128, 3, [200]),
    (8, 4, 4, 64, 5, [1000, 999]),
    (128, 16, 2, 128, 1, [700]),
    (256, 4, 2, 64, 2, [1500, 1, 513]),
    (1024, 64, 1, 64, 2, [3000, 1025]),      # largest page and G the ABI accepts: 3 row chunks
]


def _cfg(page, Hq, Hkv, d, n_q, lens, mode="shared"):
    L = max(lens)
    return synth.Config("shape", B=len(lens), Hq=Hq, Hkv=Hkv, d=d, L=L, page_size=page, n_q=n_q,
                        n_draft=2, top_k=max(1, min(64, L // 4)), n_sink=4, n_recent=16, mode=mode,
                        crit_frac=0.01)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"P{c[0]}-G{c[1] // c[2]}-d{c[3]}-nq{c[4]}")
def test_verify_select_draft(case):
    require_gpu()
    page, Hq, Hkv, d, n_q, lens = case
    cfg = _cfg(*case)
    kv = synth.make_paged_kv(cfg, seed=31, lens=lens)
    q = synth.make_queries(cfg, kv, n_q, seed=31)
    err = verify_check(cfg, kv, q)
    print(f"{case}: verify out max-abs {err:.2e}")
    # selection on the GPU's own logits, bit for bit against the CPU rule
    _, logits, _ = run_verify(cfg, kv, q)
    for mode in ("shared", "per_kv_head"):
        idx, cnt = gpu_select(logits, kv.prefix_len, Hkv, mode, cfg.top_k, cfg.n_sink, cfg.n_recent)
        assert_exact(idx, cnt, cpu_rule(logits, kv.prefix_len, Hkv, mode, cfg.top_k, cfg.n_sink,
                                         cfg.n_recent))
    # draft steps over the oracle's selection, with the verifier rows and earlier drafts as tail
    for mode in ("shared", "per_kv_head"):
        c2 = cfg.with_(mode=mode)
        sidx, scnt = selected(c2, kv, q, mode)
        for j in range(c2.n_draft):
            qd = synth.make_queries(c2, kv, 1, seed=31, tag=100 + j)
            tl = np.full(c2.B, n_q + j + 1, dtype=np.int32)
            _, _, e = sparse_check(c2, kv, qd, mode, sidx, scnt, kv.prefix_len, tl)
            print(f"{case} {mode} draft {j}: max-abs {e:.2e}")


# (page_size, Hq, Hkv, d, n_q, tree branches, blocks per row, shared blocks, prefix lengths)
BLOCK_CASES = [
    (32, 4, 2, 64, 4, 2, 3, 1, [1000, 937]),
    (128, 16, 2, 128, 8, 2, 4, 2, [3000]),
    (64, 8, 8, 128, 6, 3, 5, 3, [2500, 1999]),
]


@pytest.mark.parametrize("case", BLOCK_CASES, ids=lambda c: f"P{c[0]}-G{c[1] // c[2]}-d{c[3]}-nq{c[4]}")
def test_block_mode_shapes(case):
    """SSV block mode beyond the 16K workload's shape: head dim 64, 32- and 128-token
    blocks, one query head per KV head, and 64 q-rows per KV head (two row chunks),
    each with a tree over the verifier rows.  Blocks are drawn below the shorter
    prefix rounded up to a block, so a listed block can end past a prefix."""
    require_gpu()
    page, Hq, Hkv, d, n_q, br, kb, core, lens = case
    cfg = synth.Config("block", B=len(lens), Hq=Hq, Hkv=Hkv, d=d, L=max(lens), page_size=page, n_q=n_q,
                       n_draft=0, top_k=kb, n_sink=0, n_recent=0, mode="block", crit_frac=0.0,
                       blocks_per_row=kb, core_blocks=core, tree_branches=br)
    kv = synth.make_paged_kv(cfg, seed=41, lens=lens)
    nblk = (min(lens) + page - 1) // page          # every listed block lies below each prefix
    sets = synth.make_block_sets(cfg, nblk, seed=41)
    cnt = np.full((cfg.B, n_q, Hkv), kb, dtype=np.int32)
    q = synth.make_queries(cfg, kv, n_q, seed=41)
    tm = np.stack([synth.tree_tail_masks(n_q, br)] * cfg.B)
    tl = np.full(cfg.B, n_q, dtype=np.int32)
    _, _, e = sparse_check(cfg, kv, q, "block", sets, cnt, kv.prefix_len, tl, tm)
    print(f"{case}: block mode max-abs {e:.2e}")
