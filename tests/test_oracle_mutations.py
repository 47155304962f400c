"""Planted mistakes in the oracle must each fail a pin.

Each mutant below rewrites one expression of ``oracle/dspark_oracle.py`` into
a plausible mistake (a dropped term, a wrong sign, index or bound, a
transposed role, a wrong normaliser).  The test writes the mutated module into
a temporary copy of the ``oracle`` package, runs the CPU pin files against
that copy in a subprocess and requires the run to end in a test failure
(pytest exit status 1, not a collection error).  An unmutated copy is run
first as the control and must pass, and the copy is checked to be what the
subprocess imports.

Every mutant names the expression it replaces; the test fails loudly when
that expression no longer occurs exactly once in the oracle (a stale mutant),
so the list follows the oracle as it changes.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle")
T = os.path.join(ROOT, "tests")
PINS = {
    "core": "test_oracle_pins.py",
    "bwd": "test_oracle_backward_pins.py",
    "layer": "test_oracle_layer_pins.py",
    "loss": "test_oracle_loss_pins.py",
    "dec": "test_oracle_decode_pins.py",
}

# (name, pin group run first, expression, mistake)
MUTANTS = [
    ("bf16 decoded with a 15-bit shift", "core",
     "<< np.uint32(16)", "<< np.uint32(15)"),
    ("inverse CDF takes >= (zero-weight tokens become drawable)", "dec",
     "int(np.argmax(c > u * c[-1]))", "int(np.argmax(c >= u * c[-1]))"),
    ("window starts one position late", "core",
     "(A - W + 1 <= kv) & (kv < A)", "(A - W + 2 <= kv) & (kv < A)"),
    ("window starts one position early", "core",
     "(A - W + 1 <= kv) & (kv < A)", "(A - W <= kv) & (kv < A)"),
    ("anchor included in its own window", "core",
     "(A - W + 1 <= kv) & (kv < A)", "(A - W + 1 <= kv) & (kv <= A)"),
    ("window shifts with the query offset", "core",
     "(A - W + 1 <= kv) & (kv < A)", "(A + j - W + 1 <= kv) & (kv < A + j)"),
    ("blocks see earlier blocks", "core",
     "((kv - S) // block == n)", "((kv - S) // block <= n)"),
    ("causal inside the block", "core",
     "((kv - S) // block == n)", "((kv - S) // block == n) & (kv - S - block * n <= j)"),
    ("block positions start at A + 1", "core",
     "pos_kv.extend(int(a) + j for j in range(block))",
     "pos_kv.extend(int(a) + 1 + j for j in range(block))"),
    ("candidates keep loss_mask[S-1]", "core",
     "    lm[S - 1] = 0\n", "    pass\n"),
    ("candidates need only loss_mask[A]", "core",
     "if lm[a] == 1 and lm[a + 1] == 1:", "if lm[a] == 1:"),
    ("Fisher-Yates never reaches the last candidate", "core",
     "j = i + rng.next() % (len(C) - i)", "j = i + rng.next() % (len(C) - i - 1)"),
    ("RoPE rotates clockwise", "core",
     "y[..., 0::2] = x0 * c - x1 * s\n    y[..., 1::2] = x0 * s + x1 * c",
     "y[..., 0::2] = x0 * c + x1 * s\n    y[..., 1::2] = -x0 * s + x1 * c"),
    ("RoPE frequencies with exponent -i/d_r", "core",
     "np.power(float(base), -2.0 * i / d_r)", "np.power(float(base), -1.0 * i / d_r)"),
    ("RoPE pairs are the two halves", "core",
     "x0, x1 = x[..., 0::2], x[..., 1::2]\n    y = np.empty_like(x)",
     "x0, x1 = x[..., : d_r // 2], x[..., d_r // 2:]\n    y = np.empty_like(x)"),
    ("values use head 0's W_UV", "core",
     "V = ckv_all @ w_uv[h].T", "V = ckv_all @ w_uv[0].T"),
    ("keys drop the rope part", "core",
     "K = np.concatenate([Kc, kr_rot_all], axis=1)",
     "K = np.concatenate([Kc, 0.0 * kr_rot_all], axis=1)"),
    ("scale (d_c)^-1/2", "core",
     "return float(d_c + d_r) ** -0.5", "return float(d_c) ** -0.5"),
    ("index record pos0 off by one", "core",
     "recs[n] = (lo, len(ctx), int(anchors_row[n]), 1)",
     "recs[n] = (lo, len(ctx), int(anchors_row[n]) + 1, 1)"),
    ("dQ without the scale", "bwd",
     "dQ = scale * (dS @ K)", "dQ = (dS @ K)"),
    ("dS not centred", "bwd",
     "dS = P * (dP - np.sum(P * dP, axis=1, keepdims=True))", "dS = P * dP"),
    ("dc^KV misses the value path", "bwd",
     'dC += dKc @ x["w_uk"][h] + dV @ x["w_uv"][h]', 'dC += dKc @ x["w_uk"][h]'),
    ("dW_UV transposed role", "bwd",
     'g["dw_uv"][h] += dV.T @ C', 'g["dw_uv"][h] += 0.5 * dV.T @ C'),
    ("R^T rotates the wrong way", "bwd",
     "x[..., 0::2] = y0 * c + y1 * s\n    x[..., 1::2] = -y0 * s + y1 * c",
     "x[..., 0::2] = y0 * c - y1 * s\n    x[..., 1::2] = y0 * s + y1 * c"),
    ("RMSNorm epsilon ignored", "layer",
     "np.mean(x * x, axis=-1, keepdims=True) + eps)", "np.mean(x * x, axis=-1, keepdims=True))"),
    ("c^KV not normalised", "layer",
     "ckv_ctx=rmsnorm(kv_ctx[..., :D], f(li.g_kva), li.rms_eps)", "ckv_ctx=kv_ctx[..., :D]"),
    ("eval mask without the prefix cumprod", "loss",
     "on = on and p < S and bool(lm[b, p])", "on = p < S and bool(lm[b, p])"),
    ("confidence target 1 - L1", "loss",
     "a = np.clip(1.0 - 0.5 * l1, 0.0, 1.0)", "a = np.clip(1.0 - l1, 0.0, 1.0)"),
    ("Markov head reads the label as prev", "loss",
     "prev = ids[b, A + ks]", "prev = ids[b, A + ks + 1]"),
    ("teacher row one position late", "loss",
     "T = teacher_logits(Z[b, A + ks], w_lm)", "T = teacher_logits(Z[b, A + ks + 1], w_lm)"),
    ("labels are the inputs", "loss",
     "step_terms(L, T, ids[b, A + ks + 1], c)", "step_terms(L, T, ids[b, A + ks], c)"),
    ("loss mean over every step", "loss",
     "(float(out[k].sum() / cnt) if cnt else 0.0)",
     "(float(out[k].sum() / out[k].size) if cnt else 0.0)"),
    ("Markov bias dropped", "loss",
     "+ e @ np.asarray(w_m2, np.float64).T", "+ 0.0 * (e @ np.asarray(w_m2, np.float64).T)"),
    ("residual q - p", "dec",
     "w = np.maximum(0.0, p[j] - q[j]) if j < K else p[K]",
     "w = np.maximum(0.0, q[j] - p[j]) if j < K else p[K]"),
    ("accept ratio q / p", "dec",
     "np.exp(np.log(p[np.arange(K), x]) - np.log(q[np.arange(K), x]))",
     "np.exp(np.log(q[np.arange(K), x]) - np.log(p[np.arange(K), x]))"),
    ("ring slot off by one", "dec",
     "return np.asarray(pos) % slots", "return (np.asarray(pos) + 1) % slots"),
    ("decode window one position early", "dec",
     "ctx = np.arange(max(0, A - W + 1), A)", "ctx = np.arange(max(0, A - W), A)"),
    ("padding blocks attend to their own block", "core",
     "    if not keep_row[n]:\n        return rows\n    A = int(anchors_row[n])",
     "    if False:\n        return rows\n    A = int(anchors_row[n])"),
    ("dW_UK from the value path", "bwd",
     'g["dw_uk"][h] += dKc.T @ C', 'g["dw_uk"][h] += dV[:, :d_c].T @ C'),
    ("dK without the scale", "bwd",
     "dK = scale * (dS.T @ Q)", "dK = (dS.T @ Q)"),
    ("o_proj without the residual", "layer",
     "out[qrows] = Hd[qrows] + o2[qrows] @ f(li.w_o).T", "out[qrows] = o2[qrows] @ f(li.w_o).T"),
    ("kv_a of the draft rows from the un-normalised stream", "layer",
     "kv_blk[qrows] = h[qrows] @ f(li.w_kva).T", "kv_blk[qrows] = Hd[qrows] @ f(li.w_kva).T"),
    ("CE against the teacher's distribution", "loss",
     "ce = -np.log(p[np.arange(L.shape[0]), np.asarray(y)])",
     "ce = -np.log(q[np.arange(L.shape[0]), np.asarray(y)])"),
    ("L1 squared", "loss",
     "l1 = np.abs(p - q).sum(axis=1)", "l1 = ((p - q) ** 2).sum(axis=1)"),
    ("bonus token drawn from the last drafted position", "dec",
     "w = np.maximum(0.0, p[j] - q[j]) if j < K else p[K]",
     "w = np.maximum(0.0, p[j] - q[j]) if j < K else p[K - 1]"),
    ("temperature multiplies the logits", "dec",
     "return _softmax_rows(np.asarray(logits, np.float64) / float(temperature))",
     "return _softmax_rows(np.asarray(logits, np.float64) * float(temperature))"),
    ("target-only compares against the draft's top choice", "dec",
     "else (int(x[k]) == int(np.argmax(p[k])))", "else (int(x[k]) == int(np.argmax(q[k])))"),
    ("RMSNorm gain dropped", "layer",
     "+ eps) * np.asarray(g, np.float64)", "+ eps)"),
    ("decode block positions start at A + 1", "dec",
     "        blk = A + np.arange(BLOCK)\n", "        blk = A + 1 + np.arange(BLOCK)\n"),
    ("decode queries left unrotated", "dec",
     "Q = np.concatenate([qn[b][:, h, :], qrot[h]], axis=1)",
     "Q = np.concatenate([qn[b][:, h, :], qr[b][:, h, :]], axis=1)"),
    ("acceptance rate as a sum of maxima", "dec",
     "return np.minimum(np.asarray(p, np.float64), np.asarray(q, np.float64)).sum(axis=-1)",
     "return np.maximum(np.asarray(p, np.float64), np.asarray(q, np.float64)).sum(axis=-1)"),
    ("rejection stops one token late", "dec",
     "        if not ok:\n            j = k\n", "        if not ok:\n            j = min(k + 1, K)\n"),
    ("mask not applied (every key visible)", "core",
     "    logits = np.where(M, logits, -np.inf)\n", "    logits = np.where(M | True, logits, -np.inf)\n"),
    ("softmax without its normaliser", "core",
     "    return e / np.sum(e, axis=-1, keepdims=True)\n", "    return e\n"),
    ("keys expanded through W_UV", "core",
     "Kc = ckv_all @ w_uk[h].T            # [L, d_c]",
     "Kc = ckv_all @ w_uv[h][:w_uk.shape[1]].T            # [L, d_c]"),
    ("q_a_layernorm dropped", "layer",
     "cq = rmsnorm(h[qrows] @ f(li.w_qa).T, f(li.g_qa), li.rms_eps)", "cq = h[qrows] @ f(li.w_qa).T"),
    ("BCE target roles swapped", "loss",
     "bce = -(a * log_sig + (1.0 - a) * log_1m)", "bce = -((1.0 - a) * log_sig + a * log_1m)"),
    ("confidence head without the Markov embedding", "loss",
     "x = np.concatenate([np.asarray(h_rows, np.float64), e], axis=-1)",
     "x = np.concatenate([np.asarray(h_rows, np.float64), 0.0 * e], axis=-1)"),
]


def _source():
    with open(os.path.join(ORACLE, "dspark_oracle.py")) as f:
        return f.read()


def _copy_with(tmp, text):
    pkg = os.path.join(tmp, "oracle")
    os.makedirs(pkg, exist_ok=True)
    shutil.copy(os.path.join(ORACLE, "__init__.py"), pkg)
    with open(os.path.join(pkg, "dspark_oracle.py"), "w") as f:
        f.write(text)


def _env(tmp):
    env = dict(os.environ)
    env["PYTHONPATH"] = os.pathsep.join([tmp, ROOT, env.get("PYTHONPATH", "")])
    env["PYTHONDONTWRITEBYTECODE"] = "1"
    env.setdefault("OMP_NUM_THREADS", "1")
    return env


def _run_pins(tmp, first):
    files = [os.path.join(T, PINS[first])] + [os.path.join(T, v) for k, v in PINS.items()
                                              if k != first]
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m",
           "not gpu", *files]
    r = subprocess.run(cmd, cwd=tmp, env=_env(tmp), capture_output=True, text=True,
                       timeout=600)
    return r.returncode, r.stdout[-2000:]


def test_mutants_are_current():
    src = _source()
    stale = [name for name, _, old, _ in MUTANTS if src.count(old) != 1]
    assert not stale, f"mutant expressions not found exactly once: {stale}"


def test_every_planted_mistake_fails_a_pin():
    src = _source()
    base = tempfile.mkdtemp(prefix="oracle_mut_")
    try:
        ctrl = os.path.join(base, "control")
        _copy_with(ctrl, src)
        r = subprocess.run([sys.executable, "-c", "import oracle; print(oracle.__file__)"],
                           cwd=ctrl, env=_env(ctrl), capture_output=True, text=True)
        assert r.stdout.strip().startswith(ctrl), r.stdout + r.stderr
        code, out = _run_pins(ctrl, "core")
        assert code == 0, "unmutated copy must pass its pins:\n" + out

        def one(i):
            name, first, old, new = MUTANTS[i]
            assert src.count(old) == 1, name
            d = os.path.join(base, f"m{i}")
            _copy_with(d, src.replace(old, new))
            return name, *_run_pins(d, first)

        workers = max(1, min(8, (os.cpu_count() or 2) - 1))
        with cf.ThreadPoolExecutor(workers) as ex:
            results = list(ex.map(one, range(len(MUTANTS))))
        survived = [(n, c, o[-400:]) for n, c, o in results if c != 1]
        assert not survived, "mutants not caught by a failing pin:\n" + "\n".join(
            f"{n} (exit {c}): {o}" for n, c, o in survived)
    finally:
        shutil.rmtree(base, ignore_errors=True)
