"""Plant plausible mistakes in a copy of the oracle; the pins must catch each.

Each mutant is a textual edit of the oracle's source (a dropped term, a wrong
sign or index, a transposed operand, an off-by-one in a key set or a cache
slot).  The edited source is executed as a separate module, on the CPU; the
real oracle is untouched.
"""
import inspect
import types

import pytest

import oracle.rat_oracle as real
from tests import oracle_pins

MUTANTS = {
    "grid aligned at j mod D == 0": (
        "np.arange(D - 1, t + 1, D", "np.arange(0, t + 1, D"),
    "window starts one early": (
        "window = np.arange(max(0, t - W + 1), t + 1",
        "window = np.arange(max(0, t - W), t + 1"),
    "window drops the query's own state": (
        "window = np.arange(max(0, t - W + 1), t + 1,",
        "window = np.arange(max(0, t - W + 1), t,"),
    "empty key set falls back to own state": (
        "return np.union1d(grid, window)",
        "return np.union1d(np.union1d(grid, window), [t])"),
    "gate roles swapped": (
        "h = g * h + c * x[:, t]", "h = c * h + g * x[:, t]"),
    "initial state dropped": (
        "h = np.zeros((B, H, Dh)) if h0 is None else np.array(h0, dtype=np.float64)",
        "h = np.zeros((B, H, Dh))"),
    "sigmoid sign flipped": (
        "g = 1.0 / (1.0 + np.exp(-z))", "g = 1.0 / (1.0 + np.exp(z))"),
    "state emitted before the update": (
        "h = g * h + c * x[:, t]\n        out[:, t] = h",
        "out[:, t] = h\n        h = g * h + c * x[:, t]"),
    "softmax scale dropped": (
        "s = scale * (K @ q)", "s = (K @ q)"),
    "softmax not normalised": (
        "p /= p.sum()\n", "\n"),
    "keys used as values": (
        "return p @ V", "return p @ K"),
    "value states gated by key logits": (
        "Vt = scan(v, zv, h0v)\n    else", "Vt = scan(v, zk, h0v)\n    else"),
    "decode grid overlaps the window": (
        "sel = np.nonzero(gpos <= t - W)[0]", "sel = np.nonzero(gpos <= t - W + 1)[0]"),
    "decode grid stops one short": (
        "sel = np.nonzero(gpos <= t - W)[0]", "sel = np.nonzero(gpos < t - W)[0]"),
    "decode ring slot off by one": (
        "self.ring_k[b, h, t % W] = self.state_k[b, h]",
        "self.ring_k[b, h, (t + 1) % W] = self.state_k[b, h]"),
    "decode grid append index off by one": (
        "i = (t + 1) // D - 1\n", "i = min((t + 1) // D, self.grid_k[h].shape[1] - 1)\n"),
    "decode value state gated by key logits": (
        "gv, cv = gates(zv)", "gv, cv = gates(zk)"),
}


def _mutant(old, new):
    src = inspect.getsource(real)
    assert src.count(old) >= 1, f"mutation site not found: {old!r}"
    src = src.replace(old, new)
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, "oracle_mutant", "exec"), mod.__dict__)  # noqa: S102
    return mod


def test_real_oracle_passes_every_pin():
    assert oracle_pins.run_all(real) == []


@pytest.mark.parametrize("name", list(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    failed = oracle_pins.run_all(_mutant(old, new))
    assert failed, f"no pin catches the mutant: {name}"


# top-k block attention oracle (oracle/topk_oracle.py) against its own pins
import oracle.topk_oracle as real_topk  # noqa: E402

TOPK_MUTANTS = {
    "quest keeps only the minimum corner": (
        "np.maximum(q * kmin, q * kmax)", "q * kmin"),
    "quest takes the lower corner": (
        "np.maximum(q * kmin, q * kmax)", "np.minimum(q * kmin, q * kmax)"),
    "moba pools a sum instead of a mean": (
        "kmean[:, j] = rows.sum(axis=1) / block", "kmean[:, j] = rows.sum(axis=1)"),
    "block statistics drop the last position": (
        "rows = Kt[:, j * block:(j + 1) * block]", "rows = Kt[:, j * block:(j + 1) * block - 1]"),
    "selection keeps the lowest scores": (
        "key=lambda j: (-scores[j], j)", "key=lambda j: (scores[j], j)"),
    "ties go to the higher block": (
        "key=lambda j: (-scores[j], j)", "key=lambda j: (-scores[j], -j)"),
    "first block is a candidate": (
        "cand = list(range(1, local))", "cand = list(range(0, local))"),
    "local block is a candidate": (
        "cand = list(range(1, local))", "cand = list(range(1, local + 1))"),
    "first block not kept": (
        "blocks = sorted(set([0, local]) | set(chosen))", "blocks = sorted(set([local]) | set(chosen))"),
    "local block not kept": (
        "blocks = sorted(set([0, local]) | set(chosen))", "blocks = sorted(set([0]) | set(chosen))"),
    "local block runs past the query": (
        "hi = min((j + 1) * block - 1, t)", "hi = (j + 1) * block - 1"),
    "scores computed from the values": (
        "kmin, kmax, kmean = block_stats(Kt, block)\n    out", "kmin, kmax, kmean = block_stats(Vt, block)\n    out"),
}


def _topk_mutant(old, new):
    src = inspect.getsource(real_topk)
    assert src.count(old) >= 1, f"mutation site not found: {old!r}"
    src = src.replace(old, new).replace("from .rat_oracle import", "from oracle.rat_oracle import")
    mod = types.ModuleType("topk_mutant")
    exec(compile(src, "topk_mutant", "exec"), mod.__dict__)  # noqa: S102
    return mod


def test_real_topk_oracle_passes_every_pin():
    assert oracle_pins.run_topk(real_topk) == []


@pytest.mark.parametrize("name", list(TOPK_MUTANTS))
def test_topk_mutant_is_caught(name):
    old, new = TOPK_MUTANTS[name]
    failed = oracle_pins.run_topk(_topk_mutant(old, new))
    assert failed, f"no pin catches the mutant: {name}"


# RAT chunk-local oracle (oracle/local_oracle.py) against its own pins
import oracle.local_oracle as real_local  # noqa: E402

LOCAL_MUTANTS = {
    "restart one position late": ("if t % L == 0:\n            h = np.zeros", "if t % L == 1:\n            h = np.zeros"),
    "no restart": ("if t % L == 0:\n            h = np.zeros", "if False:\n            h = np.zeros"),
    "chunk starts from the raw input (gate forced shut)": (
        "        g, c = gates(z[:, t])\n        h = g * h + c * x[:, t]",
        "        g, c = gates(z[:, t])\n        h = x[:, t] if t % L == 0 else g * h + c * x[:, t]"),
    "own state not attended": ("return key_set(t, L, 1)", "return key_set(t, L, 0)"),
    "chunk keys one chunk apart": ("return prefill(q, None, None, None, None, L, 1,",
                                   "return prefill(q, None, None, None, None, L + 1, 1,"),
    "decode does not restart at chunk starts": ("if int(t) % L == 0:\n            cache.state_k[b] = 0.0",
                                                "if False:\n            cache.state_k[b] = 0.0"),
}


def _local_mutant(old, new):
    src = inspect.getsource(real_local)
    assert src.count(old) >= 1, f"mutation site not found: {old!r}"
    src = src.replace(old, new).replace("from .rat_oracle import", "from oracle.rat_oracle import")
    mod = types.ModuleType("local_mutant")
    exec(compile(src, "local_mutant", "exec"), mod.__dict__)  # noqa: S102
    return mod


def test_real_local_oracle_passes_every_pin():
    assert oracle_pins.run_local(real_local) == []


@pytest.mark.parametrize("name", list(LOCAL_MUTANTS))
def test_local_mutant_is_caught(name):
    old, new = LOCAL_MUTANTS[name]
    failed = oracle_pins.run_local(_local_mutant(old, new))
    assert failed, f"no pin catches the mutant: {name}"
