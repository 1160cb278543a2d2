"""Plant one plausible mistake at a time in a copy of the oracle (CPU only) and check that the
pins catch it, so a passing pin suite means something."""
import os
import types

import pytest

import oracle_pins as pins

ORACLE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")


def _load(fname, old, new, extra_subs=()):
    src = open(os.path.join(ORACLE, fname)).read()
    assert old in src, f"mutation anchor {old!r} missing from oracle/{fname}"
    src = src.replace(old, new, 1)
    for a, b in extra_subs:
        src = src.replace(a, b)
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, f"<mutant of {fname}>", "exec"), mod.__dict__)
    return mod


ATTN_MUTANTS = {
    "dropped_D_term": ("dS = P * (dP - Dc[:, None])", "dS = P * dP"),
    "dq_without_scale": ("dq[b, rows, h, :] = scale * (dS @ Kc)", "dq[b, rows, h, :] = dS @ Kc"),
    "dk_wrong_operand": ("dk[b, keys, g, :] += scale * (dS.T @ Qc)",
                         "dk[b, keys, g, :] += scale * (dS.T @ dOc)"),
    "dv_transposed_P": ("dv[b, keys, g, :] += P.T @ dOc", "dv[b, keys, g, :] += P @ dOc"),
    "gqa_modulo_map": ("return h // (H // HKV)", "return h % HKV"),
    "causal_drops_diagonal": ("vis &= j <= p", "vis &= j < p"),
    "window_off_by_one": ("vis &= j >= p - window + 1", "vis &= j >= p - window"),
    "rect_rows_top_aligned": ("p = i + (Tk - T)", "p = i"),
    "rect_offset_sign": ("p = i + (Tk - T)", "p = i + (T - Tk)"),
    "lse_log2": ("L[b, h, rows] = np.where(l > 0, m + np.log(",
                 "L[b, h, rows] = np.where(l > 0, m + np.log2("),
    "fwd_missing_scale": ("S = scale * (q[b, rows, h, :] @ k[b, keys, g, :].T)",
                          "S = (q[b, rows, h, :] @ k[b, keys, g, :].T)"),
    "key_span_drops_last_key": ("slice(int(seen[0]), int(seen[-1]) + 1)",
                                "slice(int(seen[0]), int(seen[-1]))"),
    "key_span_skips_first_key": ("slice(int(seen[0]), int(seen[-1]) + 1)",
                                 "slice(int(seen[0]) + 1, int(seen[-1]) + 1)"),
    "key_span_misaligned_mask": ("P, m, l = _softmax_rows(S, vis[:, keys])",
                                 "P, m, l = _softmax_rows(S, vis[:, :S.shape[1]])"),
    "softmax_without_max_shift_sign": ("np.exp(Sm - m[:, None])", "np.exp(Sm + m[:, None])"),
}


@pytest.mark.parametrize("name", sorted(ATTN_MUTANTS))
def test_attention_mutant_is_caught(name):
    old, new = ATTN_MUTANTS[name]
    mut = _load("attention.py", old, new)
    failures = 0
    for check in pins.ALL_FORWARD + pins.ALL_BACKWARD:
        try:
            check(mut)
        except (AssertionError, ValueError, FloatingPointError):
            failures += 1
    assert failures > 0, f"no pin caught mutant {name}"


BLOCK_MUTANTS = {
    "offset_sign": ("off = i * Bq - j * Bk", "off = j * Bk - i * Bq"),
    "offset_transposed_tiles": ("off = i * Bq - j * Bk", "off = i * Bk - j * Bq"),
    "causal_strict": ("keep &= c <= r + off", "keep &= c < r + off"),
    "walk_goes_right_first": ("below = (i + 1) * Bq - j * Bk + 1 > Bk - 1",
                              "below = (i + 1) * Bq - j * Bk + 1 >= Bk - 1"),
}


@pytest.mark.parametrize("name", sorted(BLOCK_MUTANTS))
def test_block_mutant_is_caught(name, monkeypatch):
    import oracle
    import test_oracle_blocks as tb
    old, new = BLOCK_MUTANTS[name]
    mut = _load("blocks.py", old, new,
                extra_subs=[("from .attention import visible_mask",
                             "from oracle.attention import visible_mask")])
    for attr in ("classify_blocks", "block_keep_mask", "partial_offsets_in_loop_order",
                 "triu_offset_sequence", "kv_block_range"):
        monkeypatch.setattr(oracle, attr, getattr(mut, attr))
    caught = False
    tests = [lambda: tb.test_block_masks_match_pictures(1),
             lambda: tb.test_block_masks_match_pictures(2),
             tb.test_picture_offset_claims,
             tb.test_offset_walk_known_cycles,
             lambda: tb.test_offset_walk_matches_brute_force(64, 16),
             lambda: tb.test_rebuilt_masks_match_materialised(100, 64, 16, True, 7)]
    for t in tests:
        try:
            t()
        except (AssertionError, RuntimeError):
            caught = True
    assert caught, f"no pin caught block mutant {name}"
