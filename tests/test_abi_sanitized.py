"""The C ABI layer under AddressSanitizer and UndefinedBehaviorSanitizer, with no GPU.

sub_bit_loop_amd/csrc/abi_host_check.cpp links the real lvq_abi.cpp against stub kernel
launchers that check, for every launch the ABI makes, that each buffer the kernels would
write lies inside the caller's workspace where the size query accounted for it, and that
the split plans obey the kernels' launch rules.  It draws seeded random shapes for decode
attention (per-head, grouped and multi-row routes), multi-row attention and the codebook
builder, and feeds invalid shapes that must be refused.  The stubs restate a few of the
kernels' constants (waves per workgroup, merge capacity); every workspace size the check
build reports is compared here with the real library's, so the two agree.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sub_bit_loop_amd", "csrc")
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    gxx = shutil.which("g++")
    if not gxx or not os.path.isdir(os.path.join(ROCM_INCLUDE, "hip")):
        pytest.skip("g++ or the HIP headers are not available")
    exe = str(tmp_path_factory.mktemp("abi_check") / "abi_host_check")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
           "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE,
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "lvq_abi.cpp"), os.path.join(CSRC, "abi_host_check.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    if r.returncode != 0:
        if "asan" in r.stderr.lower() and "cannot find" in r.stderr.lower():
            pytest.skip("the sanitizer runtimes are not installed")
        raise AssertionError(f"building the ABI check failed:\n{r.stderr[-4000:]}")
    return exe


@pytest.mark.parametrize("seed", [1, 2])
def test_abi_layer_under_sanitizers(checker, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([checker, str(seed), "300"], capture_output=True, text=True, timeout=600, env=env)
    summary = [l for l in r.stdout.splitlines() if l.startswith("summary:")]
    assert r.returncode == 0, f"exit {r.returncode}\n{r.stderr[-4000:]}\n{summary}"
    assert summary and summary[0].endswith("failures 0"), summary
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    n_decode = int(summary[0].split("decode calls ")[1].split(",")[0])
    assert n_decode >= 300, summary

    # the check build's workspace sizes are the real library's
    from sub_bit_loop_amd import _abi
    L = _abi.lib()
    seen = {"attn": 0, "rows": 0, "build": 0}
    for line in r.stdout.splitlines():
        f = line.split()
        if not f or f[0] not in seen:
            continue
        v = [int(x) for x in f[1:]]
        if f[0] == "attn":
            B, H, Hq, d, T, Tc, G, ns, mp, br, nip, nbp, msl, rml, nsp, need = v
            s = _abi.make_shape(B, H, Hq, d, T, Tc, G, ns, mp, br, nip, nbp, msl, rml, nsp)
            got = _abi.lvq_decode_attn_workspace_bytes(s)
        elif f[0] == "rows":
            B, NQ, H, Hq, d, T, Tc, G, ns, mp, br, nip, nbp, mpre, nsp, need = v
            s = _abi.make_rows_shape(B, NQ, H, Hq, d, T, Tc, G, ns, mp, br, nip, nbp, mpre, mpre + NQ + 1, nsp)
            got = _abi.lvq_rows_attn_workspace_bytes(s)
        else:
            T, Tc, G, S, H, d, need = v
            got = L.lvq_build_codebooks_workspace_bytes(T, Tc, G, S, H, d)
        assert got == need, (line, got)
        seen[f[0]] += 1
    assert seen["attn"] >= 250 and seen["rows"] >= 100 and seen["build"] >= 50, seen
