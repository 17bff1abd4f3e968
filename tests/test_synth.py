"""The seeded generator: determinism and the structure of what it draws."""
import numpy as np

from long_context_self_amd import synth


def test_bf16_rounding_rne():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, np.inf, 0.0, -0.0], dtype=np.float32)
    b = synth.f32_to_bf16_bits(x)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even mantissa (1.0)
    assert b[0] == 0x3F80 and b[1] == 0x3F80 and b[2] == 0x3F82
    assert b[3] == 0xC020 and b[4] == 0x7F80 and b[5] == 0 and b[6] == 0x8000
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(b)[[0, 3, 4]], np.float32([1.0, -2.5, np.inf]))


def test_deterministic_and_seed_sensitive():
    cfg = synth.CONFIGS["tiny"]
    a = synth.make_paged_kv(cfg, seed=0)
    b = synth.make_paged_kv(cfg, seed=0)
    c = synth.make_paged_kv(cfg, seed=1)
    assert a.k.tobytes() == b.k.tobytes() and a.v.tobytes() == b.v.tobytes()
    assert np.array_equal(a.block_table, b.block_table)
    assert a.k.tobytes() != c.k.tobytes()
    qa = synth.make_queries(cfg, a, 5, seed=0)
    qb = synth.make_queries(cfg, b, 5, seed=0)
    assert qa.tobytes() == qb.tobytes()


def test_paging_structure_and_poison():
    cfg = synth.CONFIGS["tiny"].with_(B=3)
    lens = [1000, 17, 333]
    kv = synth.make_paged_kv(cfg, seed=2, lens=lens)
    P = cfg.page_size
    used = []
    for b, L in enumerate(lens):
        n_tok = L + cfg.n_q + cfg.n_draft
        n_pg = (n_tok + P - 1) // P
        used.extend(kv.block_table[b, :n_pg].tolist())
        last = kv.block_table[b, n_pg - 1]
        slots = n_tok - (n_pg - 1) * P
        f = synth.bf16_bits_to_f32(kv.k[last])
        assert np.isfinite(f[:, :slots]).all()
        if slots < P:
            assert np.isnan(f[:, slots:]).all()
    assert sorted(used) == list(range(kv.num_pages))       # a permutation of all pages


def test_critical_planting():
    cfg = synth.CONFIGS["tiny"]
    kv = synth.make_paged_kv(cfg, seed=0)
    for g in range(cfg.Hkv):
        cs = kv.critical[0][g]
        assert cs.size == int(cfg.crit_frac * cfg.L) and np.unique(cs).size == cs.size
        assert cs.max() < cfg.L
    assert abs(np.linalg.norm(kv.u[0, 0]) - 1) < 1e-6


def test_block_sets_overlap():
    cfg = synth.CONFIGS["nsa_16k"]
    sets = synth.make_block_sets(cfg, n_blocks=cfg.L // cfg.page_size, seed=0)
    assert sets.shape == (cfg.B, cfg.n_q, cfg.Hkv, cfg.blocks_per_row)
    for b in range(cfg.B):
        for g in range(cfg.Hkv):
            rows = [set(sets[b, i, g].tolist()) for i in range(cfg.n_q)]
            assert len(set().union(*rows)) == 10 + 8 * 6
            for i in range(cfg.n_q):
                assert np.all(np.diff(sets[b, i, g]) > 0)
                for j in range(i):
                    assert len(rows[i] & rows[j]) == 10      # 62.5% pairwise overlap


def test_tree_masks():
    m = synth.tree_tail_masks(8, 2)
    assert [int(x) for x in m] == [0b1, 0b11, 0b111, 0b1111,
                                   0b10000, 0b110000, 0b1110000, 0b11110000]
    assert [int(x) for x in synth.chain_tail_masks(3)] == [1, 3, 7]


def test_drift_and_rewrite_keys():
    cfg = synth.CONFIGS["tiny"].with_(B=2, crit_frac=0.05)
    kv = synth.make_paged_kv(cfg, seed=3)
    old = [[c.copy() for c in row] for row in kv.critical]
    k_before = kv.k.copy()
    new = synth.drift_critical(cfg, kv, 0.2, seed=3, it=5)
    for b in range(cfg.B):
        for g in range(cfg.Hkv):
            o, n = old[b][g], new[b][g]
            assert n.size == o.size and np.all(np.diff(n) > 0)          # same size, sorted, distinct
            assert n.min() >= 0 and n.max() < kv.prefix_len[b]
            assert np.setdiff1d(o, n).size == int(round(0.2 * o.size))  # the moved fraction
    rows, bits = synth.rewrite_keys(cfg, kv, new, seed=3, it=5)
    flat_new, flat_old = kv.k.reshape(-1, cfg.d), k_before.reshape(-1, cfg.d)
    assert np.array_equal(flat_new[rows], bits)
    changed = np.any(flat_new != flat_old, axis=1)
    assert set(np.nonzero(changed)[0].tolist()) <= set(rows.tolist())
    # joined rows carry the planted direction, left rows do not
    for b in range(cfg.B):
        for g in range(cfg.Hkv):
            joined = np.setdiff1d(new[b][g], old[b][g])
            left = np.setdiff1d(old[b][g], new[b][g])
            kf = synth.bf16_bits_to_f32(
                kv.k[kv.block_table[b, joined // cfg.page_size], g, joined % cfg.page_size])
            kl = synth.bf16_bits_to_f32(
                kv.k[kv.block_table[b, left // cfg.page_size], g, left % cfg.page_size])
            assert (kf @ kv.u[b, g]).mean() > (kl @ kv.u[b, g]).mean() + 1.5
            assert kv.critical[b][g] is new[b][g]
