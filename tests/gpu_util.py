"""Helpers for the GPU parity tests (test-side only)."""
import functools

import numpy as np
import torch

import synth

# Layer-output bar: max-abs error <= 2e-2 and relative Frobenius error <= 5e-3
# against the float64 oracle.
MAX_ABS = 2e-2
REL_FROB = 5e-3

# Small shapes: each spans several tiles with ragged tails; together they cover
# GQA ratios 1/2/4/8, head_dim 64/128, B = 2, D = 1, one-row chunks (c = 1),
# chunk lengths that are not multiples of the attention row block (c = 96,
# 24), MLP shards whose width is not a multiple of 64 (F/D = 176, 96), and
# attention blocks long enough to be split along the keys.
SWEEP = {
    "mha_d2_r1": (1, 256, 2, 1, 256, 4, 4, 64, 768),
    "gqa4_dh128_d4_r2": (1, 512, 4, 2, 256, 16, 4, 128, 512),
    "gqa8_b2_c96": (2, 384, 2, 1, 128, 16, 2, 64, 256),
    "ffn_tail_d4_r3": (1, 256, 4, 3, 192, 8, 4, 64, 704),
    "d1": (1, 128, 1, 0, 128, 2, 2, 64, 256),
    "c1_d8_r5": (1, 16, 8, 5, 64, 8, 8, 64, 512),
    "c24_generic_reorder": (1, 96, 2, 0, 128, 4, 2, 64, 192),
    "wide_tiles_dh128": (1, 1024, 2, 0, 512, 8, 8, 128, 1536),
    "gqa2_b2_dh128_c80": (2, 320, 2, 1, 256, 8, 4, 128, 640),
    # few 128-row blocks with long key ranges: attention splits blocks into
    # key pieces and merges them
    "split_keys_dh128": (1, 4096, 2, 0, 128, 2, 2, 128, 256),
    "split_keys_gqa_b2": (2, 2048, 2, 1, 128, 4, 2, 64, 256),
    # degree 8, a middle rank: both chunks split into key pieces and paired
    "split_keys_d8_r5": (1, 8192, 8, 5, 128, 8, 8, 128, 256),
}


def dims_of(shape):
    return synth.Dims(*shape)


@functools.lru_cache(maxsize=None)
def inputs_for(shape, sigma=0.02, seed=101):
    return synth.make_inputs(dims_of(shape), sigma, seed)


def errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = got - ref
    return float(np.abs(diff).max()), float(np.linalg.norm(diff) / np.linalg.norm(ref))


def assert_close(got, ref, max_abs=MAX_ABS, rel_frob=REL_FROB, what=""):
    ma, rf = errors(got, ref)
    print(f"  {what}: max_abs={ma:.3e} rel_frob={rf:.3e}", flush=True)
    assert np.all(np.isfinite(got)), what
    assert ma <= max_abs and rf <= rel_frob, f"{what}: max_abs {ma:.3e} rel_frob {rf:.3e}"


def sample_rows(T, c, n_extra=6, seed=0):
    """First/last rows of both zigzag chunks plus a few seeded others."""
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 2, c - 1, c, c + 1, c + 2, T - 1]
    extra = rng.choice(T, size=min(n_extra, T), replace=False).tolist()
    return np.array(sorted(set(r for r in fixed + extra if 0 <= r < T)), dtype=np.int64)


def f16_bits_to_f64(t):
    return t.cpu().numpy().view(np.float16).astype(np.float64)


def dev():
    return torch.device("cuda:0")


def block_edge_rows(T, c, rb=128, seed=0, n_extra=4):
    """The first and last row of every rb-row block of both halves of the
    rank's rows (each attention row block, with its split and paired key
    pieces, is then compared at least twice), plus sample_rows'."""
    rows = set(sample_rows(T, c, n_extra=n_extra, seed=seed).tolist())
    for half0, half1 in ((0, c), (c, T)):
        for b0 in range(half0, half1, rb):
            rows.add(b0)
            rows.add(min(b0 + rb, half1) - 1)
    return np.array(sorted(rows), dtype=np.int64)


class tuning:
    """Context manager: kernel-choice overrides through tsp_set_tuning, reset
    to the default dispatch on exit."""

    def __init__(self, **knobs):
        self.knobs = knobs

    def __enter__(self):
        from folded_tensor_sequence_amd import binding as B
        for k, v in self.knobs.items():
            B.tsp_set_tuning(k, v)
        return self

    def __exit__(self, *exc):
        from folded_tensor_sequence_amd import binding as B
        B.reset_tuning()
        return False
