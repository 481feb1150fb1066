"""Mutation check of the oracle's pins (CPU only).

Each case plants one plausible mistake in a copy of the oracle source (never
in the file itself), runs tests/test_oracle_pins.py against that copy in a
fresh interpreter, and requires the pins to fail.  A control run of the
unmodified copy must pass.  So every pinned reading is shown to be held by
at least one pin, not only to agree with it.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle", "msa_oracle.py")

# (what the mistake is, exact text of the oracle, replacement)
MUTANTS = [
    ("queries at the first len_q positions",
     "return np.arange(len_kv - len_q, len_kv, dtype=np.int64)",
     "return np.arange(0, len_q, dtype=np.int64)"),
    ("causal mask off by one",
     "dots[key_pos[None, :] > pos[r0:r1, None]] = NEG_INF",
     "dots[key_pos[None, :] >= pos[r0:r1, None]] = NEG_INF"),
    ("mean pooling instead of max pooling",
     "S[g, r0:r1, :nb] = dots.reshape(r1 - r0, nb, block_size).max(axis=2)",
     "S[g, r0:r1, :nb] = np.where(np.isneginf(dots), 0.0, dots).reshape(r1 - r0, nb, block_size)"
     ".mean(axis=2)"),
    ("ties to the higher block",
     "order = np.lexsort((cand, -S[g, t, :J]))",
     "order = np.lexsort((-cand, -S[g, t, :J]))"),
    ("one free pick too few",
     "kept = sorted(int(j) for j in cand[order[:top_k - 1]]) + [J]",
     "kept = sorted(int(j) for j in cand[order[:top_k - 2]]) + [J]"),
    ("forced block of the previous position",
     "            J = int(pos[t] // block_size)\n            if J <= top_k - 1:\n"
     "                kept = list(range(J + 1))",
     "            J = int(max(pos[t] - 1, 0) // block_size)\n            if J <= top_k - 1:\n"
     "                kept = list(range(J + 1))"),
    ("vectorised selection: ties to the higher block",
     "kb = gt | (eq & (np.cumsum(eq, axis=1) <= need))",
     "kb = gt | (eq & (np.cumsum(eq[:, ::-1], axis=1)[:, ::-1] <= need))"),
    ("softmax scale dropped",
     "z = scale * (kg @ qf[t, hs].T)",
     "z = (kg @ qf[t, hs].T)"),
    ("LSE without the max",
     "lse[t, hs] = m + np.log(l)",
     "lse[t, hs] = np.log(l)"),
    ("strided head-to-group map",
     "hs = slice(g * hpg, (g + 1) * hpg)",
     "hs = slice(g, H, G)"),
    ("block mass not averaged over the group's heads",
     "mass[g, t, i] += a[at:at + sk.size].sum() / hpg",
     "mass[g, t, i] += a[at:at + sk.size].sum()"),
    ("KL in the reverse direction",
     "kl[g, t] = float((p[pos_p] * (np.log(p[pos_p]) - logq[pos_p])).sum())",
     "kl[g, t] = float((q * (logq - np.log(np.maximum(p, 1e-300)))).sum())"),
    ("KL gradient with the wrong sign",
     "grad[g, t, slots] = q * p.sum() - p",
     "grad[g, t, slots] = p - q * p.sum()"),
    ("arg-max in fp32, channel order",
     "    dots = _f64(k_rows) @ _f64(q_row)\n",
     "    qq = np.asarray(_f64(q_row), np.float32)\n"
     "    kk = np.asarray(_f64(k_rows), np.float32)\n"
     "    dots = np.zeros(kk.shape[0], np.float32)\n"
     "    for c in range(qq.shape[0]):\n"
     "        dots = (dots + qq[c] * kk[:, c]).astype(np.float32)\n"),
    ("arg-max ties to the higher key",
     "return int(np.argmax(dots))",
     "return int(len(dots) - 1 - np.argmax(dots[::-1]))"),
    ("attention backward without the D term",
     "dz = a * (dp - do[t, h] @ out)",
     "dz = a * dp"),
    ("dk without the softmax scale",
     "gk = scale * np.outer(dz, qf[t, h])",
     "gk = np.outer(dz, qf[t, h])"),
    ("coarse keys summed instead of averaged",
     "return k[:nfull * span].reshape(nfull, span, G, di).mean(axis=1)",
     "return k[:nfull * span].reshape(nfull, span, G, di).sum(axis=1)"),
    ("coarse ties to the higher chunk",
     "order = np.lexsort((cand_chunks, -coarse[g, t, :cJ]))",
     "order = np.lexsort((-cand_chunks, -coarse[g, t, :cJ]))"),
    ("current chunk's blocks not scored",
     "blocks = [c * S + s for c in keep for s in range(S)] + list(range(cJ * S, J))",
     "blocks = [c * S + s for c in keep for s in range(S)]"),
    ("recall counting the forced block",
     "r = set(int(x) for x in ref[g, t] if 0 <= x < J)",
     "r = set(int(x) for x in ref[g, t] if 0 <= x <= J)"),
]


def _run_pins(src: str) -> tuple:
    """Runs the pins against an oracle with source `src` in a scratch tree;
    returns (pytest exit status, last line of its output)."""
    with tempfile.TemporaryDirectory(prefix="oracle_mutant_") as tmp:
        os.makedirs(os.path.join(tmp, "oracle"))
        shutil.copy(os.path.join(ROOT, "oracle", "__init__.py"), os.path.join(tmp, "oracle"))
        with open(os.path.join(tmp, "oracle", "msa_oracle.py"), "w") as f:
            f.write(src)
        shutil.copy(os.path.join(ROOT, "workloads.py"), tmp)  # the seeded input generator
        os.makedirs(os.path.join(tmp, "tests"))
        for name in ("conftest.py", "test_oracle_pins.py"):
            shutil.copy(os.path.join(ROOT, "tests", name), os.path.join(tmp, "tests"))
        shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(tmp, "tests", "golden"))
        env = {k: v for k, v in os.environ.items() if k != "PYTHONPATH"}
        env["PYTHONDONTWRITEBYTECODE"] = "1"
        env["OMP_NUM_THREADS"] = "1"
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                            os.path.join("tests", "test_oracle_pins.py")],
                           cwd=tmp, env=env, capture_output=True, text=True, timeout=600)
        lines = r.stdout.strip().splitlines()
        return r.returncode, lines[-1] if lines else r.stderr[-300:]


def test_every_planted_mistake_fails_a_pin():
    with open(ORACLE) as f:
        src = f.read()
    for name, old, new in MUTANTS:
        assert src.count(old) == 1, f"mutation site of '{name}' not found exactly once"
    jobs = [("control", src)] + [(name, src.replace(old, new)) for name, old, new in MUTANTS]
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        results = dict(zip([j[0] for j in jobs], ex.map(lambda j: _run_pins(j[1]), jobs)))
    rc, last = results.pop("control")
    assert rc == 0, f"the unmodified oracle copy fails its pins: {last}"
    survivors = [f"{n}: {last}" for n, (rc, last) in results.items() if rc == 0]
    broken = [f"{n}: exit {rc}, {last}" for n, (rc, last) in results.items() if rc not in (0, 1)]
    assert not broken, "mutants that did not run: " + "; ".join(broken)
    assert not survivors, "mistakes no pin catches: " + "; ".join(survivors)
