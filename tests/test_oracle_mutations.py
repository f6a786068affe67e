"""The oracle's pins must catch plausible mistakes: each case below plants one
mistake in a copy of the oracle (on the CPU, in a temporary directory) and
checks that the pin tests fail against the mutated copy."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "dsa_oracle.py")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

muts = [
 ("var unbiased", "var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)", "var = ((x - mu) ** 2).sum(axis=-1, keepdims=True) / (x.shape[-1] - 1)"),
 ("no beta", "* gamma + beta", "* gamma"),
 ("no gamma", "* gamma + beta", "+ beta"),
 ("no eps", "np.sqrt(var + eps)", "np.sqrt(var)"),
 ("no mean", "return (x - mu) / np.sqrt", "return (x) / np.sqrt"),
 ("relu abs", "np.maximum(0.0, scale * dots)", "np.abs(scale * dots)"),
 ("scale outside", "(w[r][None, :] * np.maximum(0.0, scale * dots))", "(w[r][None, :] * np.maximum(0.0, dots))"),
 ("causal off by one", "+ kp - 1 <= row_pos", "+ kp <= row_pos"),
 ("no validity", "np.asarray(pool_valid_b, dtype=bool) &", ""),
 ("softmax over channels", "m = logits.max(axis=1, keepdims=True)       # per pool and channel\n            e = np.exp(logits - m)\n            a = e / e.sum(axis=1, keepdims=True)", "m = logits.max(axis=2, keepdims=True)\n            e = np.exp(logits - m)\n            a = e / e.sum(axis=2, keepdims=True)"),
 ("ape by token", "logits = gate[b][t] + ape[None, :, :]", "logits = gate[b][t] + ape[t % kp]"),
 ("no ape", "logits = gate[b][t] + ape[None, :, :]", "logits = gate[b][t]"),
 ("anchor zero", "f_b = int(idx[0])", "f_b = 0"),
 ("partial pool counted", "return f_b, (T_b - f_b) // kp", "return f_b, -(-(T_b - f_b) // kp)"),
 ("validity first slot only", "pool_valid[b, p] = np.all(valid[b][t] != 0, axis=1)", "pool_valid[b, p] = valid[b][t[:, 0]] != 0"),
 ("tie index desc", "order = np.lexsort((cand, -vals))", "order = np.lexsort((-cand, -vals))"),
 ("ascending score", "order = np.lexsort((cand, -vals))", "order = np.lexsort((cand, vals))"),
 ("no slot offset", "tok[r, j * kp:(j + 1) * kp] = pool_start[b, p] + np.arange(kp)", "tok[r, j * kp:(j + 1) * kp] = pool_start[b, p]"),
 ("expand wrong seq", "b = int(row_seq[r])\n        for j in", "b = 0\n        for j in"),
 ("mla wrong seq", "b = int(row_seq[r])\n        ids", "b = 0\n        ids"),
 ("mla no scale", "logits = sm_scale * (q_lat[r] @ V.T)", "logits = (q_lat[r] @ V.T)"),
 ("lse no max", "lse[i] = (m + np.log(l))[:, 0]", "lse[i] = (np.log(l))[:, 0]"),
 ("mla no norm", "out[i] = (e @ V) / l", "out[i] = (e @ V)"),
 ("w heads reversed", "s = (w[r][None, :]", "s = (w[r][::-1][None, :]"),
 ("w row 0 for all rows", "s = (w[r][None, :]", "s = (w[0][None, :]"),
 ("scores rows seq", "b = int(row_seq[r])\n        if b not in normed", "b = 0\n        if b not in normed"),
 ("empty ids", "ids = token_ids[r][token_ids[r] >= 0]", "ids = np.abs(token_ids[r])"),
 ("fp8 bias 8", "(1.0 + m / 8.0) * np.ldexp(1.0, e - 7)", "(1.0 + m / 8.0) * np.ldexp(1.0, e - 8)"),
 ("fp8 no subnormals", "np.where(e == 0, (m / 8.0) * 2.0 ** -6,", "np.where(e == 0, 0.0 * m,"),
 ("fp8 no nan", "mag = np.where((e == 15) & ((c & 7) == 7), np.nan, mag)", "pass"),
 ("fp8 scale ignored", "return vals * f64(kv_scale).reshape(-1, 1)", "return vals"),
 ("page row from page start", "out[r, c] = pg * page_size + t % page_size", "out[r, c] = pg * page_size"),
 ("page by token not table", "pg = int(bt[b, t // page_size])", "pg = t // page_size"),
 ("page table of sequence 0", "pg = int(bt[b, t // page_size])", "pg = int(bt[0, t // page_size])"),
 ("out-of-range page kept", "if 0 <= pg < num_pages:", "if True:"),
]


@pytest.mark.parametrize("name,old,new", muts, ids=[m[0] for m in muts])
def test_pins_catch_planted_mistake(name, old, new, tmp_path):
    base = open(SRC).read()
    assert old in base, "mutation anchor no longer in the oracle: " + name
    d = tmp_path / "oracle"
    d.mkdir()
    (d / "__init__.py").write_text("")
    (d / "dsa_oracle.py").write_text(base.replace(old, new, 1))
    env = dict(os.environ, PYTHONPATH=f"{tmp_path}:{ROOT}")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", PINS],
                       env=env, capture_output=True, text=True, cwd=str(tmp_path), timeout=300)
    assert r.returncode != 0, f"pins did not catch: {name}\n{r.stdout[-2000:]}"
