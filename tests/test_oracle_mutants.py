"""Planted mistakes in the oracle are caught by its pins.

Each case loads a copy of an oracle module's source with one plausible slip
planted in it (a dropped term, a wrong operand, a transposed product, a wrong
mask, log base, sign, a generator constant), on the CPU, and checks that the
pins fail on the copy while they pass on the unmodified source.  The pins
used here are the same independent references as in test_oracle_pins.py and
test_dropout_oracle_pins.py: the pure-Python brute force, splitmix64's
published outputs and the keep decisions they fix, the keep rate, and the
unbiasedness of inverted dropout.
The oracle files themselves are never modified.
"""

import math
import pathlib
import types

import numpy as np
import pytest

import oracle.attention as attention_ok
from tests.test_dropout_oracle_pins import _brute as brute_dropout
from tests.test_oracle_pins import _brute as brute_attention

ROOT = pathlib.Path(__file__).resolve().parents[1]


def load(relpath, old=None, new=None):
    """A fresh module from the file's source, with `old` replaced by `new`."""
    src = (ROOT / relpath).read_text()
    if old is not None:
        assert src.count(old) == 1, old
        src = src.replace(old, new)
    mod = types.ModuleType("oracle_copy")
    if relpath.endswith("dropout.py"):
        # the relative import of the attention helpers, resolved by hand
        line = "from .attention import _check_head, _scores, _softmax_rows\n"
        assert line in src
        src = src.replace(line, "")
        mod.__dict__.update(_check_head=attention_ok._check_head, _scores=attention_ok._scores,
                            _softmax_rows=attention_ok._softmax_rows)
    exec(compile(src, str(ROOT / relpath), "exec"), mod.__dict__)
    return mod


def attention_pins_pass(m):
    rng = np.random.default_rng(5)
    for S, hd, causal in ((5, 4, True), (5, 4, False), (7, 3, True)):
        q, k, v, do = (rng.standard_normal((S, hd)) for _ in range(4))
        got = m.attention_forward_head(q, k, v, 0.7, causal) + m.attention_backward_head(q, k, v, do, 0.7, causal)
        out, lse, dq, dk, dv, dref = got
        b_out, b_lse, b_dq, b_dk, b_dv, b_dref = brute_attention(q, k, v, do, 0.7, causal)
        for a, b in ((out, b_out), (lse, b_lse), (dq, b_dq), (dk, b_dk), (dv, b_dv), (dref, b_dref)):
            if a.shape != b.shape or not np.allclose(a, b, rtol=0, atol=1e-10):
                return False
    return True


def dropout_pins_pass(m):
    golden = 0x9E3779B97F4A7C15
    states = np.array([0, golden, (2 * golden) % 2**64], dtype=np.uint64)
    if [int(x) for x in m.splitmix64(states)] != [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]:
        return False
    # keep decisions at indices whose u the published outputs fix
    from tests.test_dropout_oracle_pins import _keep_cases
    for seed, index, u in _keep_cases():
        u32 = np.float32(u)
        idx = np.array([index], dtype=np.uint64)
        if not (m.keep_mask(seed, idx, float(u32))[0]
                and not m.keep_mask(seed, idx, float(np.nextafter(u32, np.float32(1))))[0]):
            return False
    n, p = 1 << 16, 0.3
    keep = m.keep_mask(2024, np.arange(n, dtype=np.uint64), p)
    if abs(keep.sum() - n * (1 - p)) > 5 * math.sqrt(n * p * (1 - p)):
        return False
    rng = np.random.default_rng(6)
    S, hd, seed, bh = 6, 3, 4242, 1
    q, k, v, do = (rng.standard_normal((S, hd)) for _ in range(4))
    idx = np.array([[(bh * S + i) * S + j for j in range(S)] for i in range(S)], dtype=np.uint64)
    M = m.keep_mask(seed, idx, p).astype(np.float64) / (1 - p)
    if not np.array_equal(M, m.probs_mask(seed, p, bh, S, 0, S)):
        return False
    out, _ = m.attention_dropout_forward_head(q, k, v, 0.7, True, p, seed, bh)
    dq, dk, dv, _ = m.attention_dropout_backward_head(q, k, v, do, 0.7, True, p, seed, bh)
    for a, b in zip((out, dq, dk, dv), brute_dropout(q, k, v, do, 0.7, True, M)):
        if not np.allclose(a, b, rtol=1e-12, atol=1e-12):
            return False
    # inverted dropout is unbiased: the mean over seeds tends to the plain output
    plain, _ = attention_ok.attention_forward_head(q, k, v, 0.7, True)
    outs = np.stack([m.attention_dropout_forward_head(q, k, v, 0.7, True, 0.5, s, 0)[0] for s in range(400)])
    err = np.abs(outs.mean(0) - plain)
    return bool(np.all(err <= 5 * outs.std(0) / math.sqrt(len(outs)) + 1e-12))


def test_unmodified_sources_pass():
    assert attention_pins_pass(load("oracle/attention.py"))
    assert dropout_pins_pass(load("oracle/dropout.py"))


ATTENTION_SLIPS = {
    "mask off by one": ("s = np.where(cols > rows, _NEG_INF, s)", "s = np.where(cols > rows + 1, _NEG_INF, s)"),
    "mask direction": ("s = np.where(cols > rows, _NEG_INF, s)", "s = np.where(cols < rows, _NEG_INF, s)"),
    "log base 2": ("return e / l[:, None], mx + np.log(l)", "return e / l[:, None], mx + np.log2(l)"),
    "unsafe softmax dropped max": ("return e / l[:, None], mx + np.log(l)", "return e / l[:, None], np.log(l)"),
    "dropped scale in the backward": ("        g = dsm * scale\n", "        g = dsm\n"),
    "dropped Jacobian term": ("dsm = p * (dp - rs[:, None])", "dsm = p * dp"),
    "Jacobian sign": ("dsm = p * (dp - rs[:, None])", "dsm = p * (rs[:, None] - dp)"),
    "wrong operand in dQ": ("dq[r0:r1] = g @ k", "dq[r0:r1] = g @ v"),
    "untransposed P in dV": ("dv += p.T @ do_rows", "dv += p @ do_rows"),
    "wrong operand in dP": ("dp = do_rows @ v.T", "dp = do_rows @ k.T"),
}


@pytest.mark.parametrize("slip", sorted(ATTENTION_SLIPS))
def test_attention_slip_is_caught(slip):
    old, new = ATTENTION_SLIPS[slip]
    assert not attention_pins_pass(load("oracle/attention.py", old, new)), slip


DROPOUT_SLIPS = {
    "generator constant": ("GOLDEN = np.uint64(0x9E3779B97F4A7C15)", "GOLDEN = np.uint64(0x9E3779B97F4A7C17)"),
    "generator shift": ("z = (z ^ (z >> np.uint64(30))) * _M1", "z = (z ^ (z >> np.uint64(31))) * _M1"),
    "keep test reversed": ("return u >= np.float32(p)", "return u < np.float32(p)"),
    "no inverted scaling": ("return keep_mask(seed, idx, p).astype(np.float64) / (1.0 - p)",
                            "return keep_mask(seed, idx, p).astype(np.float64)"),
    "mask left out of dV": ("dv += (pr * m).T @ do_rows", "dv += pr.T @ do_rows"),
    "mask left out of dP": ("dp = m * (do_rows @ v.T)", "dp = do_rows @ v.T"),
    "dropped scale in the dropout backward": ("g = pr * (dp - rs[:, None]) * scale", "g = pr * (dp - rs[:, None])"),
    "index not multiplied by golden": ("key = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) ^ (idx * GOLDEN)",
                                       "key = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) ^ idx"),
    "addition in place of XOR": ("key = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) ^ (idx * GOLDEN)",
                                 "key = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + (idx * GOLDEN)"),
    "low 24 bits in place of the top 24": ("u = (h >> np.uint64(40)).astype(np.float32)",
                                           "u = (h & np.uint64(0xFFFFFF)).astype(np.float32)"),
    "index rows and keys swapped": ("idx = (np.uint64(bh) * np.uint64(S) + i) * np.uint64(S) + j",
                                    "idx = (np.uint64(bh) * np.uint64(S) + j) * np.uint64(S) + i"),
}


@pytest.mark.parametrize("slip", sorted(DROPOUT_SLIPS))
def test_dropout_slip_is_caught(slip):
    old, new = DROPOUT_SLIPS[slip]
    assert not dropout_pins_pass(load("oracle/dropout.py", old, new)), slip
