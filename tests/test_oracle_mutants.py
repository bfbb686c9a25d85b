"""The oracle's pins must reject plausible mistakes: each case below plants one mistake in
a temporary copy of the oracle (on the CPU) and runs the oracle's pin tests against it;
every planted mistake must make at least one pin fail."""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "attamba_oracle.py")
PINS = ["test_oracle_segment.py", "test_oracle_scan.py", "test_oracle_attention.py",
        "test_oracle_decode.py", "test_oracle_proj.py", "test_oracle_backward.py",
        "test_oracle_block.py", "test_oracle_stack.py"]

MUTANTS = [
    ("decay uses the previous step size", "decay = np.exp(delta[k][:, None] * A)",
     "decay = np.exp(delta[max(k - 1, 0)][:, None] * A)"),
    ("decay sign", "decay = np.exp(delta[k][:, None] * A)",
     "decay = np.exp(-delta[k][:, None] * A)"),
    ("skip term dropped", "y[k] = h @ np.asarray(Cm[t], np.float64) + D * x[t]",
     "y[k] = h @ np.asarray(Cm[t], np.float64)"),
    ("no reset at chunk start", "            h = np.zeros_like(A)\n        k = t - t_begin",
     "            pass\n        k = t - t_begin"),
    ("Bm read for Cm", "y[k] = h @ np.asarray(Cm[t], np.float64) + D * x[t]",
     "y[k] = h @ np.asarray(Bm[t], np.float64) + D * x[t]"),
    ("input term without step size", "inject = (delta[k] * x[t])", "inject = (x[t])"),
    ("window one token wider", "visible = ie[j] | ((i - j) < L)",
     "visible = ie[j] | ((i - j) <= L)"),
    ("M_train sees earlier chunks", "visible = visible | (tc[j] == tc[i])",
     "visible = visible | (tc[j] <= tc[i])"),
    ("mask not causal", "return (j <= i) & visible", "return visible"),
    ("P times K instead of V", "out[live, h, :] = (p[live] @ v[:, h, :])",
     "out[live, h, :] = (p[live] @ k[:, h, :])"),
    ("score scale dropped", "s = (q[:, h, :] @ k[:, h, :].T) * scale",
     "s = (q[:, h, :] @ k[:, h, :].T)"),
    ("boundary state at chunk start", "return y[np.asarray(chunk_cu[1:], dtype=np.int64) - 1]",
     "return y[np.asarray(chunk_cu[:-1], dtype=np.int64)]"),
    ("decode window one token wider", "st.recent = [r for r in st.recent if r[0] > i - L]",
     "st.recent = [r for r in st.recent if r[0] >= i - L]"),
    ("decode boundary inside window", "keys = [r for r in st.bounds if r[0] < w]",
     "keys = [r for r in st.bounds if r[0] <= w]"),
    ("decode without state reset", "        st.h_k = np.zeros_like(st.h_k)\n", "        pass\n"),
    ("softplus sign", "return np.logaddexp(0.0, z)", "return np.logaddexp(0.0, -z)"),
    ("LSE without the max", "lse[h, live] = mx[live] + np.log(denom[live])",
     "lse[h, live] = np.log(denom[live])"),
    ("chunk end flag at chunk start", "is_end[chunk_cu[q + 1] - 1] = 1", "is_end[chunk_cu[q]] = 1"),
    ("projection weight not transposed", "return x @ w.T", "return x @ w"),
    ("projection output features reversed", "return x @ w.T", "return (x @ w.T)[:, ::-1]"),
    ("projection with a dropped input feature", "return x @ w.T", "return x[:, 1:] @ w[:, 1:].T"),
    ("first chunk not shortened by the offset", "return [t for t in range(n) if t == 0 or (t - o) % P == 0]",
     "return [t for t in range(n) if t % P == 0]"),
    ("backward state gradient not decayed", "            dh = dh * e\n", "            pass\n"),
    ("backward softmax without the row term", "ds = p * (dp - (dp * p).sum(axis=1, keepdims=True))",
     "ds = p * dp"),
    ("backward softplus derivative dropped", "dz = ddelta * sig[t]", "dz = ddelta"),
    ("backward dA without the step size", "g[\"dA\"] += de * e * delta[t][:, None]",
     "g[\"dA\"] += de * e"),
    ("backward key gradient from dS instead of dS^T", "dk[:, h, :] = scale * (ds.T @ q[:, h, :])",
     "dk[:, h, :] = scale * (ds @ q[:, h, :])"),
    ("convolution taps reversed", "acc = acc + w[:, k] * x[s]", "acc = acc + w[:, K - 1 - k] * x[s]"),
    ("convolution does not restart at chunk starts", "                if s >= a:\n", "                if s >= 0:\n"),
    ("convolution bias dropped", "            acc = b.copy()", "            acc = np.zeros(d)"),
    ("SiLU replaced by the logistic function", "return v / (1.0 + np.exp(-v))", "return 1.0 / (1.0 + np.exp(-v))"),
    ("gate applied without SiLU", "return y if z is None else y * silu(z)", "return y if z is None else y * z"),
    ("bf16 rounding keeps one bit too many", "return np.ldexp(np.round(m * 256.0), e - 8)",
     "return np.ldexp(np.round(m * 512.0), e - 9)"),
    ("stack feeds the unrounded output on", "        x = round_to_bf16(res[\"out\"].reshape(T, d))",
     "        x = res[\"out\"].reshape(T, d)"),
    ("stack layers all at the first offset", "res = kvssm_forward(inp, seq_cu, H, hd, P, first_layer + l, L, mode)",
     "res = kvssm_forward(inp, seq_cu, H, hd, P, first_layer, L, mode)"),
    ("block skip term on the raw input", "    y, _ = selective_scan(xc, dt, dt_bias, A, Bm, Cm, D, chunk_cu)\n    return y if z",
     "    y, _ = selective_scan(xc, dt, dt_bias, A, Bm, Cm, D, chunk_cu)\n    y = y + D * (np.asarray(x) - xc)\n    return y if z"),
]


def _run(tmp, i, name, old, new):
    src = open(SRC).read()
    assert old in src, name
    tree = os.path.join(tmp, f"m{i}")
    os.makedirs(tree)
    for sub in ("oracle", "workloads", "tests"):
        shutil.copytree(os.path.join(ROOT, sub), os.path.join(tree, sub),
                        ignore=shutil.ignore_patterns("__pycache__"))
    with open(os.path.join(tree, "oracle", "attamba_oracle.py"), "w") as f:
        f.write(src.replace(old, new, 1))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *[os.path.join("tests", p) for p in PINS]],
                       cwd=tree, capture_output=True, text=True, timeout=600)
    return name, r.returncode


def test_pins_reject_planted_mistakes(tmp_path):
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        results = list(ex.map(lambda a: _run(str(tmp_path), *a),
                              [(i, *m) for i, m in enumerate(MUTANTS)]))
    survived = [name for name, rc in results if rc == 0]
    assert not survived, f"planted mistakes not caught by any pin: {survived}"
