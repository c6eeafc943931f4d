"""The synthetic input generators: sequence selection, target-row alignment, and the
all-accept verify inputs (CPU only)."""
import numpy as np

from block_drafter_draft_amd import workloads as wl


def test_sequence_selection_matches_the_full_batch():
    for c, attn in ((1, True), (3, False)):
        cfg = wl.CONFIGS[c]
        full = wl.make_step_inputs(cfg, iset=1, with_attention=attn, with_codebooks=False)
        for b in sorted({0, cfg.B - 1, cfg.B // 2}):
            one = wl.make_step_inputs(cfg, iset=1, with_attention=attn, with_codebooks=False,
                                      seqs=[b])
            for name in ("ctx_len", "draft", "target", "gate", "anchor", "temperature"):
                np.testing.assert_array_equal(getattr(one, name), getattr(full, name)[b:b + 1],
                                              err_msg=f"config {c} seq {b} {name}")
            for name in ("q", "k_ring", "conv_x", "conv_delta"):
                for a, f in zip(getattr(one, name), getattr(full, name)):
                    np.testing.assert_array_equal(a, f[b:b + 1], err_msg=f"{name}")


def test_target_row_r_is_built_around_draft_row_r_plus_1():
    # proposal r + 1 comes from draft row r + 1 and is verified by target row r
    cfg = wl.CONFIGS[1]                    # f32 logits: target = base + noise exactly
    d = wl.draft_logits(cfg)
    t = wl.target_rows(cfg, d)
    N = cfg.N
    for r in range(N):
        aligned = np.corrcoef(t[0, r], d[0, r + 1])[0, 1]
        same = np.corrcoef(t[0, r], d[0, r])[0, 1]
        # var(draft) = 3, var(noise) = 1: correlation sqrt(3/4) = 0.866 when aligned
        assert aligned > 0.8 and abs(same) < 0.15, (r, aligned, same)
    bonus = wl.bonus_draft_row(cfg)
    assert np.corrcoef(t[0, N], bonus[0, 0])[0, 1] > 0.8
    assert max(abs(np.corrcoef(t[0, N], d[0, r])[0, 1]) for r in range(cfg.P)) < 0.15


def test_all_accept_inputs_accept_every_proposal(orc):
    for c, seqs in ((1, None), (2, None), (3, [0, 5]), (5, [0, 1, 2, 3])):
        cfg = wl.CONFIGS[c]
        vi = wl.all_accept_verify_inputs(cfg, iset=0, seqs=seqs)
        B = vi.tokens.shape[0]
        # every proposal is one of its slot's candidates, at its slot
        np.testing.assert_array_equal(
            np.take_along_axis(vi.cand_idx, vi.slot[..., None], axis=2)[..., 0], vi.tokens)
        for step in (0, 3):
            n, out, st = orc.verify(vi.target.reshape(-1), B, cfg.N, cfg.P * cfg.V, cfg.V,
                                    cfg.V, vi.tokens, vi.cand_idx, vi.q, vi.slot,
                                    vi.temperature, cfg.seed, step)
            assert np.all(n == cfg.N) and not st.any(), (c, n, st)
            np.testing.assert_array_equal(out[:, :cfg.N], vi.tokens)
