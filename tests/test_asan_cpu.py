"""Host AddressSanitizer runs of the host code: the fp64 oracle and the host
packer (pack_plan.cpp), each built with -fsanitize=address and exercised in
a child process (the sanitizer runtime has to be loaded first, so the child
starts with it preloaded).

The oracle runs every function on small inputs with the edge cases the GPU
tests use (empty and single-token sequences, every conv width and d_state,
carried states, the step map, error-scale mode); the packer runs every
strategy on ordinary, empty, exact-fit and over-long inputs. Any heap or
stack overrun, use after free or double free fails the test.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def asan_build(tmp_path_factory):
    rt = _asan_runtime()
    if rt is None or shutil.which("g++") is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    d = tmp_path_factory.mktemp("asan")
    import oracle
    flags = ("-fsanitize=address", "-fno-omit-frame-pointer", "-g")
    orc = oracle.build(str(d / "liboracle_asan.so"), extra_flags=flags)
    pk = str(d / "libpack_asan.so")
    subprocess.run(["g++", "-O1", "-std=c++17", "-fPIC", "-shared", *flags, "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "selective_state_space_varlen_amd", "csrc", "pack_plan.cpp"), "-o", pk],
                   check=True)
    return rt, orc, pk


def _run_child(rt, code):
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=23",
               PYTHONPATH=ROOT)
    r = subprocess.run([sys.executable, "-c", textwrap.dedent(code)], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=600)
    assert "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, r.stderr[-4000:]
    return r.stdout


def test_oracle_under_asan(asan_build):
    rt, orc_path, _ = asan_build
    out = _run_child(rt, f"""
        import numpy as np
        import oracle, synth
        orc = oracle.Oracle({orc_path!r})
        rng = np.random.default_rng(0)
        cases = [([4, 2, 3, 7], 8, 4, 4), ([1], 3, 1, 1), ([0, 5, 0, 1, 9], 7, 2, 2), ([33, 1, 64], 5, 16, 3),
                 ([0], 2, 8, 4)]
        n = 0
        for lengths, D, N, W in cases:
            cu = synth.cu_seqlens_of(lengths)
            T = int(cu[-1])
            pos, head = orc.pack_indices(cu, T)
            x, z, dout = (rng.standard_normal((T, D)) for _ in range(3))
            w, b = rng.uniform(-0.5, 0.5, (D, W)), rng.standard_normal(D)
            delta = rng.uniform(0.01, 0.2, (T, D))
            A, B, C = -rng.uniform(0.5, 2.0, (D, N)), rng.standard_normal((T, N)), rng.standard_normal((T, N))
            Dp, bias = rng.standard_normal(D), rng.standard_normal(D) * 0.3
            nseq = len(lengths)
            h0, dhT = rng.standard_normal((nseq, D, N)), rng.standard_normal((nseq, D, N))
            xc0, dxcT = rng.standard_normal((nseq, W - 1, D)), rng.standard_normal((nseq, W - 1, D))
            for threads in (1, 3):
                for scales in (False, True):
                    ctx = orc.error_scales() if scales else __import__("contextlib").nullcontext()
                    with ctx:
                        v, u = orc.conv_fwd(x, w, b, pos, True, threads=threads)
                        orc.scan_fwd(u, delta, A, B, C, Dp, z, pos, threads=threads)
                        orc.scan_bwd(u, delta, A, B, C, Dp, z, pos, dout, threads=threads, delta_bias=bias,
                                     delta_softplus=True, gate_floor=0.05)
                        orc.scan_bwd(u, delta, A, B, C, None, None, pos, dout, threads=threads)
                        orc.conv_bwd(x, w, None, pos, dout, False, threads=threads)
                        orc.conv_fwd_state(x, w, b, cu, xc0, threads=threads)
                        orc.conv_bwd_state(x, w, b, cu, dout, xc0, dxcT, threads=threads)
                        orc.scan_fwd_state(u, delta, A, B, C, Dp, z, cu, h0=h0, threads=threads)
                        orc.scan_bwd_state(u, delta, A, B, C, Dp, z, cu, dout, h0=h0, dhT=dhT, threads=threads,
                                           delta_bias=bias, delta_softplus=True, gate_floor=0.05)
                        if T:
                            orc.forward(x, w, b, delta, A, B, C, Dp, z, cu, threads=threads)
                            orc.backward(x, w, b, delta, A, B, C, Dp, z, cu, dout, threads=threads)
                    n += 1
        print("oracle runs", n)
    """)
    assert "oracle runs 20" in out


def test_packer_under_asan(asan_build):
    rt, _, pk_path = asan_build
    out = _run_child(rt, f"""
        import ctypes
        import numpy as np
        lib = ctypes.CDLL({pk_path!r})
        vp = ctypes.c_void_p
        lib.varlen_pack_plan.restype = ctypes.c_int
        lib.varlen_pack_plan.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                         vp, vp, vp, vp, vp, vp]

        def plan(lengths, cap, strategy, window):
            ln = np.ascontiguousarray(lengths, dtype=np.int32)
            n = ln.size
            order, bounds, cu = np.empty(n, np.int32), np.empty(n + 1, np.int32), np.empty(n + 1, np.int32)
            mx, npk, pad = np.empty(max(n, 1), np.int32), np.zeros(1, np.int32), np.zeros(1, np.int64)
            p = lambda a: a.ctypes.data_as(vp)
            return lib.varlen_pack_plan(p(ln), n, cap, strategy, window, p(order), p(bounds), p(cu), p(mx),
                                        p(npk), p(pad))

        rng = np.random.default_rng(1)
        calls = 0
        for strategy in (0, 1):
            for window in (1, 2, 16, 1000):
                for lengths, cap in ((rng.integers(1, 4097, 300), 4096), ([], 4096), ([4096, 4096, 1], 4096),
                                     ([0, 0, 5], 8), ([7], 7), (rng.integers(0, 65, 2000), 64)):
                    assert plan(lengths, cap, strategy, window) == 0
                    calls += 1
                assert plan([5, 9], 8, strategy, window) != 0  # longer than a pack
                assert plan([3, -1], 8, strategy, window) != 0  # negative length
                calls += 2
        assert plan([1, 2], 0, 0, 1) != 0
        assert plan([1, 2], 8, 7, 1) != 0
        print("packer calls", calls + 2)
    """)
    assert "packer calls 66" in out
