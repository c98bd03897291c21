"""The oracle's dimension contract, and the whole oracle pin suite under ASan/UBSan.

The oracle accepts any 1 <= k <= E <= 256 (more than the GPU library's top-8 limit), so
its per-row working arrays are sized for 256 entries and every function that takes k
checks it. These pins cover the k > 8 range, where a per-row array sized for the
"top eight" of "0 train-infer mismatch ...", "The router: matching expert ids and
weights" would overflow:

* the scored router's softmax mode selects and weights exactly as the plain router
  (same selection key, same FP32 softmax, same left-to-right renormaliser), bitwise;
* the router backward at k = 16 agrees with float64 autograd of the definition
  (full softmax, top-k at the router's own choice, renormalised weights);
* the rank combine at k = 16 with one rank is the plain slot-order combine, bitwise;
* bad dimensions are rejected, not silently mis-computed.

The last test compiles ``oracle/moe_oracle.c`` with AddressSanitizer and
UndefinedBehaviorSanitizer (host code only) and runs the CPU pin suites against that
build in a child process, so an out-of-bounds access or undefined operation anywhere in
the pinned paths fails the test.
"""
import os
import shutil
import subprocess
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _logits(T, E, seed, ties=False):
    rng = np.random.default_rng(seed)
    if ties:
        return rng.integers(0, 3, (T, E)).astype(np.float32)
    return rng.normal(0, 2, (T, E)).astype(np.float32)


@pytest.mark.parametrize("k", [9, 16, 32])
@pytest.mark.parametrize("ties", [False, True])
def test_scored_softmax_equals_plain_router_beyond_eight(orc, k, ties):
    lg = _logits(64, 32, 11 + k, ties)
    idx, w, mass, err = orc.route_from_logits(lg, k)
    r = orc.route_scored(lg, k, "softmax")
    assert err == 0 and r["err"] == 0
    assert r["idx"].tobytes() == idx.tobytes()
    assert r["w"].tobytes() == w.tobytes()
    assert r["prob_mass"].tobytes() == mass.tobytes()
    # the selection is the first k of the order (logit desc, id asc)
    order = np.lexsort((np.tile(np.arange(32), (64, 1)), -lg), axis=1)[:, :k]
    assert (idx == order).all()
    # renormalised weights sum to 1 within k roundings
    assert np.abs(w.astype(np.float64).sum(1) - 1).max() <= k * 2.0 ** -23


def test_router_backward_beyond_eight_matches_float64_autograd(orc):
    T, E, k, d = 24, 32, 16, 8
    rng = np.random.default_rng(5)
    x = rng.normal(0, 1, (T, d)).astype(np.float32)
    wr = rng.normal(0, 1 / np.sqrt(d), (E, d)).astype(np.float32)
    logits = orc.router_logits(x, wr, None, "f32")
    dw = rng.normal(0, 1, (T, k)).astype(np.float32)
    br = orc.backward_router(logits, dw, x, wr, "f32")
    sel, _, _, _ = orc.route_from_logits(logits, k)
    lt = torch.tensor(logits, dtype=torch.float64, requires_grad=True)
    p = torch.softmax(lt, 1)
    ps = torch.gather(p, 1, torch.as_tensor(sel, dtype=torch.long))
    wsel = ps / ps.sum(1, keepdim=True)
    (wsel * torch.tensor(dw, dtype=torch.float64)).sum().backward()
    ref = lt.grad.numpy()
    err = np.abs(br["dl"].astype(np.float64) - ref).max() / np.abs(ref).max()
    assert err <= 2e-5, err
    # dl sums to zero per token (softmax), within FP32 rounding
    assert np.abs(br["dl"].astype(np.float64).sum(1)).max() <= 1e-5 * np.abs(br["dl"]).max()


def test_rank_combine_beyond_eight_single_rank_is_plain_combine(orc):
    rng = np.random.default_rng(6)
    T, k, d, E = 40, 16, 24, 32
    y = rng.normal(0, 1, (T * k, d)).astype(np.float32)
    inv = rng.permutation(T * k).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    idx = np.argsort(rng.random((T, E)), 1)[:, :k].astype(np.int32)
    for dtype in ("bf16", "f32"):
        parts, out = orc.combine_ranks(y, inv, w, idx, E, 1, dtype)
        plain = orc.combine(y, inv, w, dtype)
        assert out.tobytes() == plain.tobytes() == parts[0].tobytes()
    # R = E: every rank owns one expert; a rank's partial is its one slot's w * y, rounded
    parts, out = orc.combine_ranks(y, inv, w, idx, E, E, "f32")
    for t in range(0, T, 7):
        for j in range(k):
            e = idx[t, j]
            want = (np.float32(w[t, j]) * y[inv[t * k + j]]).astype(np.float32)
            assert parts[e, t].tobytes() == want.tobytes()


def test_bad_dimensions_are_rejected(orc):
    lg = _logits(4, 8, 1)
    with pytest.raises(ValueError):
        orc.route_from_logits(lg, 9)
    with pytest.raises(ValueError):
        orc.route_scored(lg, 9, "softmax")
    with pytest.raises(ValueError):
        orc.backward_router(lg, np.zeros((4, 9), np.float32), np.zeros((4, 2), np.float32),
                            np.zeros((8, 2), np.float32), "f32")
    y = np.zeros((8, 2), np.float32)
    inv = np.arange(8, dtype=np.int32)
    w = np.ones((4, 2), np.float32)
    idx = np.tile(np.arange(2, dtype=np.int32), (4, 1))
    with pytest.raises(ValueError):
        orc.combine_ranks(y, inv, w, idx, 8, 3, "f32")          # 3 does not divide 8
    with pytest.raises(ValueError):
        orc.combine_ranks(y, inv, w, idx, 8, 16, "f32")         # more ranks than experts


_PIN_SUITES = ["tests/test_oracle_pins.py", "tests/test_oracle_bounds.py",
               "tests/test_router_variants.py", "tests/test_rank_reduction.py",
               "tests/test_backward_oracle.py", "tests/test_placement.py"]


def _asan_runtime():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(os.environ.get("MOE_ORACLE_LIB") is not None,
                    reason="already running against another oracle build")
def test_oracle_pins_under_address_and_undefined_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    asan = _asan_runtime()
    if asan is None:
        pytest.skip("libasan not available")
    lib = str(tmp_path / "libmoe_oracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                    "-std=c11", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-shared", "-fPIC", "-o", lib,
                    os.path.join(ROOT, "oracle", "moe_oracle.c"), "-lm"], check=True)
    env = dict(os.environ)
    pre = env.get("LD_PRELOAD")
    env.update(MOE_ORACLE_LIB=lib, LD_PRELOAD=asan + (":" + pre if pre else ""),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-m", "not gpu",
                        "-p", "no:cacheprovider", *_PIN_SUITES], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr, tail
    assert "runtime error" not in r.stderr, tail
