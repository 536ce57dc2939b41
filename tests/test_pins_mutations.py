"""The oracle's pins catch plausible mistakes (CPU): each case plants one mistake in a
scratch copy of oracle/ (a dropped term, a wrong sign, index, axis or constant) and
runs the oracle's own tests against that copy, which must then fail. The GPU path
is not involved; the planted mistakes live only in the temporary copy."""
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (what the mistake is, text in oracle/kvq_oracle.py, replacement)
MUTATIONS = [
    ("butterfly difference sign", "v[..., 1, :] = (a - b).astype(_F32)", "v[..., 1, :] = (b - a).astype(_F32)"),
    ("rotation not normalized", "return (y * _F32(1.0 / math.sqrt(128.0))).astype(_F32)", "return y.astype(_F32)"),
    ("2^b levels instead of 2^b - 1", "levels = _F32(2 ** bits - 1)", "levels = _F32(2 ** bits)"),
    ("codes from the fp32 scale, not the stored fp16 one",
     "inv = (_F32(1.0) / np.where(zero_scale, _F32(1.0), s16_32)).astype(_F32)",
     "inv = (_F32(1.0) / np.where(zero_scale, _F32(1.0), s32)).astype(_F32)"),
    ("ties rounded up instead of to even", "r = np.rint(prod).astype(_F32)",
     "r = np.floor(prod + _F32(0.5)).astype(_F32)"),
    ("no clamp to [0, 2^b - 1]", "r = np.clip(r, _F32(0), levels)", "pass"),
    ("zero-point from the maximum", "z16 = mn.astype(_F16)", "z16 = mx.astype(_F16)"),
    ("value scales tiled instead of repeated (dequantize_block)",
     "vs_full = np.repeat(vs.astype(np.float64), GROUP, axis=1)",
     "vs_full = np.tile(vs.astype(np.float64), (1, GROUP))"),
    ("value scales tiled instead of repeated (attention)",
     "vs_full = np.repeat(self.vs.astype(np.float64), self.G, axis=2)",
     "vs_full = np.tile(self.vs.astype(np.float64), (1, 1, self.G))"),
    ("residual rule ignores the sink", "return G * (max(0, T - o - R) // G)", "return G * (max(0, T - R) // G)"),
    ("residual rule off by one", "return G * (max(0, T - o - R) // G)", "return G * (max(0, T - o - R + 1) // G)"),
    ("rotary sine sign", "return np.concatenate([a * c - b * s, b * c + a * s], axis=1)",
     "return np.concatenate([a * c + b * s, b * c - a * s], axis=1)"),
    ("rotary frequency exponent over 128", "theta = float(base) ** (-np.arange(half, dtype=np.float64) / half)",
     "theta = float(base) ** (-np.arange(half, dtype=np.float64) / x.shape[-1])"),
    ("scores not scaled", "s = (q @ k.T) * scale", "s = (q @ k.T)"),
    ("softmax normalized over all heads", "p = p / p.sum(axis=1, keepdims=True)", "p = p / p.sum()"),
    ("keys quantized per token", "kc, ks, kz = quantize_uniform(kg, self.bits, axis=1)",
     "kc, ks, kz = quantize_uniform(kg, self.bits, axis=2)"),
    ("values quantized per channel", "vc, vs, vz = quantize_uniform(vg, self.bits, axis=3)",
     "vc, vs, vz = quantize_uniform(vg, self.bits, axis=1)"),
    ("sink rotated at position 1", "pos = np.concatenate([pos, [0]])", "pos = np.concatenate([pos, [1]])"),
    ("query not rotated", "return wht128_fp32(q.astype(_F32)).astype(np.float64)", "return q.astype(np.float64)"),
    ("default scale 1/D", "self.scale = softmax_scale if softmax_scale else 1.0 / math.sqrt(head_dim)",
     "self.scale = softmax_scale if softmax_scale else 1.0 / head_dim"),
    ("query heads interleaved over kv-heads", "rows = slice(h * ratio, (h + 1) * ratio)",
     "rows = slice(h, self.Hq, self.Hkv)"),
]
# Not listed: dropping the explicit all-zero codes of a group whose fp16 scale is 0.
# It changes nothing: with the unit reciprocal used there, (x - z) rounds to code 0
# for every such group (its range is below one fp16 subnormal step times 2^b - 1).


def _run_mutated(base, name, old, new):
    """Copy oracle/ and the tests into base, plant one mistake, run the oracle tests;
    returns (name, pytest exit status, tail of its output)."""
    os.makedirs(base)
    for d in ("oracle", "tests", "kvq_workloads"):
        shutil.copytree(os.path.join(ROOT, d), os.path.join(base, d),
                        ignore=shutil.ignore_patterns("__pycache__"))
    shutil.copy(os.path.join(ROOT, "pytest.ini"), base)
    src = os.path.join(base, "oracle", "kvq_oracle.py")
    with open(src) as f:
        text = f.read()
    if text.count(old) != 1:
        return name, -1, f"mutation site not found once: {old!r}"
    with open(src, "w") as f:
        f.write(text.replace(old, new))
    tests = sorted(os.path.join(base, "tests", f) for f in os.listdir(os.path.join(base, "tests"))
                   if f.startswith("test_oracle") and f.endswith(".py"))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"]
                       + tests, cwd=base, capture_output=True, text=True, timeout=600)
    return name, r.returncode, (r.stdout[-1500:] + r.stderr[-500:])


def test_every_planted_mistake_fails_the_oracle_tests(tmp_path):
    # one scratch copy per mistake, several pytest runs at a time
    from concurrent.futures import ThreadPoolExecutor
    workers = max(1, min(6, (os.cpu_count() or 2) - 1))
    with ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(lambda im: _run_mutated(str(tmp_path / f"m{im[0]}"), *im[1]), enumerate(MUTATIONS)))
    survivors = [(name, rc, out) for name, rc, out in results if rc != 1]
    assert not survivors, "\n\n".join(f"{name} (exit {rc}):\n{out}" for name, rc, out in survivors)
