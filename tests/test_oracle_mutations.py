"""The oracle's pins catch plausible mistakes in the oracle itself (CPU only).

Each case copies `oracle/` and `tests/` into a temporary directory, plants one
slip in the copy of an oracle module (a rounding mode, a dropped or extra
term, a wrong sign, index, axis or transpose), and runs that module's pin
tests there in a fresh interpreter: they must fail.  The unmodified copy must
pass, so a failure is the planted slip's doing.  Nothing under the real
`oracle/` is written.  The exhaustive encoder scan and the whole-layer
forward pin are left out of these runs to keep them short; the pins that do
the catching are the closed forms, invariants and brute-force checks.
"""

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
E, Q, G, F, L, C = ("test_oracle_e4m3.py", "test_oracle_quant.py", "test_oracle_gemm.py", "test_oracle_fused.py",
                    "test_oracle_layer.py", "test_oracle_compare.py")

# (module, original text, planted text, pin files that must catch it)
MUTATIONS = [
    ("e4m3.py", "n = np.rint(a / spacing)", "n = np.floor(a / spacing + 0.5)", [E, Q]),           # ties away
    ("e4m3.py", "binade = np.maximum(ex - 1, -6)", "binade = np.maximum(ex - 1, -7)", [E, Q]),    # subnormal edge
    ("e4m3.py", "m = np.minimum(n * spacing, E4M3_MAX)", "m = n * spacing", [E, Q]),               # no saturation
    ("e4m3.py", "sign = np.signbit(v).astype(np.uint8) << 7", "sign = (v < 0).astype(np.uint8) << 7", [E, Q]),
    ("e4m3.py", "(e - 10).astype(np.int32)", "(e - 11).astype(np.int32)", [E, G]),                 # decode bias
    ("e4m3.py", "sub = f * _SUB_QUANTUM", "sub = f * _SUB_QUANTUM * 2", [E, G]),
    ("quant.py", "s = (amax / np.float32(448.0)).astype(np.float32)",
     "s = (amax * np.float32(1 / 448.0)).astype(np.float32)", [Q]),                                # reciprocal scale
    ("quant.py", "quotient = (x / s).astype(np.float32)",
     "quotient = (x * (np.float32(1.0) / s)).astype(np.float32)", [Q]),                            # reciprocal quotient
    ("quant.py", "codes = np.where(s == 0, np.uint8(0), codes).astype(np.uint8)", "codes = codes.astype(np.uint8)",
     [Q]),                                                                                         # zero groups
    ("quant.py", "amax = np.max(np.abs(blk), axis=1, keepdims=True)", "amax = np.max(blk, axis=1, keepdims=True)",
     [Q]),
    ("quant.py", "np.asarray(x_bits, dtype=np.uint16).T)", "np.asarray(x_bits, dtype=np.uint16))", [Q, G]),
    ("quant.py", "np.repeat(np.asarray(block_scales), GROUP, axis=0)",
     "np.repeat(np.asarray(block_scales).T, GROUP, axis=0)", [Q, G]),                              # block index
    ("quant.py", "amax = np.float32(np.max(np.abs(blk)))", "amax = np.float32(np.max(np.abs(blk[0])))", [Q]),
    ("quant.py", "c0, c1 = g * GROUP, min((g + 1) * GROUP, C)", "c0, c1 = g * GROUP, min((g + 1) * GROUP + 1, C)",
     [Q]),                                                                                         # group edge
    ("gemm.py", "np.asarray(row_scales, dtype=np.float64), GROUP",
     "np.asarray(row_scales, dtype=np.float64)[:, ::-1], GROUP", [G]),                            # scale index
    ("gemm.py", "    y = a @ b.T\n", "    y = (a @ b.T) * (1 + 2.0 ** -20)\n", [G]),
    ("gemm.py", "    y = a @ b.T\n    bnd = (np.abs(a) @ np.abs(b).T)", "    y = a @ b.T\n    bnd = np.abs(a @ b.T)",
     [G]),                                                                                         # error budget
    ("fused.py", "h = g / (1.0 + np.exp(-g)) * u", "h = u / (1.0 + np.exp(-u)) * g", [F]),
    ("fused.py", "np.sqrt(np.mean(x * x, axis=1) + float(np.float32(eps)))",
     "(np.sqrt(np.mean(x * x, axis=1)) + float(np.float32(eps)))", [F]),
    ("fused.py", "y = x * rstd[:, None] * gamma[None, :]", "y = x * rstd[:, None]", [F]),
    ("layer.py", "rot = np.concatenate([-t[..., half:], t[..., :half]], axis=-1)",
     "rot = np.concatenate([t[..., half:], -t[..., :half]], axis=-1)", [L]),                        # RoPE sign
    ("layer.py", "sc = q @ k.transpose(0, 2, 1) / np.sqrt(HEAD_DIM)", "sc = q @ k.transpose(0, 2, 1)", [L]),
    ("layer.py", "np.tril(np.ones((s, s), dtype=bool))", "np.triu(np.ones((s, s), dtype=bool))", [L]),
    ("layer.py", "k, v = np.repeat(k, rep, axis=0), np.repeat(v, rep, axis=0)",
     "k, v = np.tile(k, (rep, 1, 1)), np.tile(v, (rep, 1, 1))", [L]),                             # GQA heads
    ("layer.py", "g, u = gu[:, :INTER], gu[:, INTER:]", "u, g = gu[:, :INTER], gu[:, INTER:]", [L]),
    ("layer.py", "np.mean(x * x, axis=-1, keepdims=True) + EPS", "np.sum(x * x, axis=-1, keepdims=True) + EPS", [L]),
    ("layer.py", "return _bf(g / (1.0 + np.exp(-g)) * u)", "return _bf(_bf(g / (1.0 + np.exp(-g))) * u)", [L]),
    ("layer.py", "return _bf(_bf(gate / (1.0 + np.exp(-gate))) * up)", "return _bf(gate / (1.0 + np.exp(-gate)) * up)",
     [L]),                                                                                         # SwiGLU roundings
    ("compare.py", "a, b = a.view(width), b.view(width)", "pass", [C]),                          # value compare
    ("compare.py", "if a.shape != b.shape or a.dtype != b.dtype:", "if a.shape != b.shape:", [C]),
]


def _run(module, old, new, files):
    d = tempfile.mkdtemp(prefix="oracle_mutation_")
    try:
        skip = shutil.ignore_patterns("__pycache__")
        shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(d, "oracle"), ignore=skip)
        shutil.copytree(os.path.join(ROOT, "tests"), os.path.join(d, "tests"), ignore=skip)
        os.symlink(os.path.join(ROOT, "blockwise_fp8_linear_quant_amd"), os.path.join(d, "blockwise_fp8_linear_quant_amd"))
        if module is not None:
            path = os.path.join(d, "oracle", module)
            src = open(path).read()
            assert src.count(old) == 1, (module, old)
            with open(path, "w") as f:
                f.write(src.replace(old, new))
        cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
               "-k", "not exhaustive and not residual_paths"] + [os.path.join("tests", t) for t in files]
        r = subprocess.run(cmd, cwd=d, capture_output=True, text=True, timeout=600)
        return r.returncode, (r.stdout + r.stderr)[-400:]
    finally:
        shutil.rmtree(d, ignore_errors=True)


@pytest.fixture(scope="module")
def results():
    with ThreadPoolExecutor(4) as ex:
        base = ex.submit(_run, None, None, None, [E, Q, G, F, L, C])
        muts = list(ex.map(lambda m: _run(*m), MUTATIONS))
    return base.result(), muts


def test_unmodified_copy_passes(results):
    (rc, tail), _ = results
    assert rc == 0, tail


@pytest.mark.parametrize("i", range(len(MUTATIONS)), ids=[f"{m[0]}:{m[2][:40]}" for m in MUTATIONS])
def test_planted_slip_is_caught(results, i):
    rc, tail = results[1][i]
    assert rc == 1, (MUTATIONS[i][:3], tail)
