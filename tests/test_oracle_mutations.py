"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
the pins reject every one: a dropped factor, a wrong sign, a transposed
operand, a wrong mask direction, the inverse rescale printed on one page."""
import math
import os
import types

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _mutant(module_file, old, new, name):
    path = os.path.join(ROOT, "oracle", module_file)
    with open(path) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType(name)
    mod.__package__ = "oracle"
    mod.__file__ = path
    exec(compile(src.replace(old, new), path, "exec"), mod.__dict__)
    return mod


def _five():
    import json
    with open(os.path.join(ROOT, "tests", "golden", "five_position.json")) as f:
        g = json.load(f)
    return [np.array(g[x], dtype=np.float64) for x in ("Q", "K", "V", "G")]


def _fd_check(mod):
    """Finite differences of L = sum(O o G) on the five-position example."""
    q, k, v, g = _five()
    scale = 1 / math.sqrt(2)
    dq, dk, dv, *_ = mod.head_backward(q, k, v, g, scale, True, check_d_identity=False)
    h = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        arrs = [q.copy(), k.copy(), v.copy()]
        x = arrs[which]
        for idx in np.ndindex(*x.shape):
            x0 = x[idx]
            x[idx] = x0 + h
            lp = float(np.sum(mod.head_forward(*arrs, scale, True)[0] * g))
            x[idx] = x0 - h
            lm = float(np.sum(mod.head_forward(*arrs, scale, True)[0] * g))
            x[idx] = x0
            if abs((lp - lm) / (2 * h) - grad[idx]) > 1e-7:
                return False
    return True


def _closed_forms(mod):
    """Row-0 closed form, scale = 0 uniform average, causal LSE count."""
    q, k, v, g = _five()
    o, lse = mod.head_forward(q, k, v, 1 / math.sqrt(2), True)
    if abs(lse[0] - (0.2 * 0.3 - 0.3 * 0.5) / math.sqrt(2)) > 1e-14 or np.abs(o[0] - v[0]).max() > 1e-14:
        return False
    o0, l0 = mod.head_forward(q, k, v, 0.0, True)
    for i in range(5):
        if np.abs(o0[i] - v[: i + 1].mean(axis=0)).max() > 1e-14 or abs(l0[i] - math.log(i + 1)) > 1e-14:
            return False
    return True


def _all_pins_pass(mod):
    return _fd_check(mod) and _closed_forms(mod)


def test_unmutated_oracle_passes_the_harness():
    from oracle import attention
    assert _all_pins_pass(attention)


MUTATIONS = [
    ("attention.py", "dk += scale * (ds.T @ q[r])", "dk += (ds.T @ q[r])", "dK without scale"),
    ("attention.py", "dq[r] = scale * (ds @ k)", "dq[r] = (ds @ k)", "dQ without scale"),
    ("attention.py", "ds = p * (dp - d_r[:, None])", "ds = p * (dp + d_r[:, None])", "sign of D"),
    ("attention.py", "ds = p * (dp - d_r[:, None])", "ds = p * dp", "dropped D term"),
    ("attention.py", "dp = do[r] @ v.T", "dp = 0.5 * (do[r] @ v.T)", "scaled dP"),
    ("attention.py", "dv += p.T @ do[r]", "dv += p.T @ do[r][:, ::-1]", "transposed operand columns in dV"),
    ("attention.py", "vis &= keys[None, :] <= rows[:, None]\n", "vis &= keys[None, :] < rows[:, None]\n", "causal diagonal excluded"),
    ("attention.py", "vis &= keys[None, :] <= rows[:, None]\n", "vis &= keys[None, :] >= rows[:, None]\n", "causal mask inverted"),
    ("attention.py", "s = scale * (q_rows @ k.T)", "s = (q_rows @ k.T) / max(scale, 1e-300)", "scale divides"),
    ("attention.py", "lse = np.where(dead, -np.inf, m_safe + np.log(np.where(dead, 1.0, denom)))",
     "lse = np.where(dead, -np.inf, np.log(np.where(dead, 1.0, denom)))", "LSE without max"),
]


@pytest.mark.parametrize("module_file,old,new,label", MUTATIONS, ids=[m[3] for m in MUTATIONS])
def test_planted_mistake_is_caught(module_file, old, new, label):
    mod = _mutant(module_file, old, new, "oracle_mutant")
    assert not _all_pins_pass(mod), f"pins did not catch: {label}"


def _tiling_invariant_holds(tiled_mod):
    from oracle import attention
    rng = np.random.default_rng(0)
    n, d = 23, 4
    q, k, v, g = (rng.standard_normal((n, d)) * 1.5 for _ in range(4))
    for br, bc in ((4, 4), (5, 3), (8, 16)):
        o_t, l_t = tiled_mod.tiled_forward(q, k, v, 0.5, br, bc, True)
        dq_t, dk_t, dv_t = tiled_mod.tiled_backward(q, k, v, g, 0.5, br, bc, True)
        dq, dk, dv, o, lse, _ = attention.head_backward(q, k, v, g, 0.5, True)
        if not (np.allclose(o_t, o, rtol=1e-12, atol=1e-13) and np.allclose(l_t, lse, rtol=1e-12)
                and np.allclose(dq_t, dq, atol=1e-12) and np.allclose(dk_t, dk, atol=1e-12)):
            return False
    return True


TILED_MUTATIONS = [
    ("acc = alpha[:, None] * acc + p_tilde @ v[cols]", "acc = acc / np.where(alpha == 0, 1.0, alpha)[:, None] + p_tilde @ v[cols]",
     "inverse rescale of the accumulator"),
    ("ell = alpha * ell + p_tilde.sum(axis=1)", "ell = ell + p_tilde.sum(axis=1)", "denominator not rescaled"),
    ("dvec = np.sum(do * o, axis=1)", "dvec = np.zeros(o.shape[0])", "D dropped in the tiled backward"),
]


@pytest.mark.parametrize("old,new,label", TILED_MUTATIONS, ids=[m[2] for m in TILED_MUTATIONS])
def test_planted_tiling_mistake_is_caught(old, new, label):
    from oracle import tiled
    assert _tiling_invariant_holds(tiled)
    mod = _mutant("tiled.py", old, new, "oracle_tiled_mutant")
    assert not _tiling_invariant_holds(mod), f"tiling invariant did not catch: {label}"
