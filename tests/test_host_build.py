"""Host-only builds of the native code, run on the CPU (no GPU needed):

- the C ABI layer (yoco_api.cpp) with test-only launchers, under
  AddressSanitizer and UndefinedBehaviorSanitizer: valid calls reach the
  launchers with the promised parameters, launcher failures become
  YOCO_ERR_LAUNCH, rejected calls launch nothing, and the decode's 32-bit row
  offsets hold at the largest accepted cache length (tests/host_build/abi_driver.cpp);
- the division by invariant integers the streaming kernels use
  (tests/host_build/fastdiv_check.cpp), against plain division;
- every LDS address the pipelined prefill forms (prefill_layout.h, through
  tests/host_build/prefill_layout_check.cpp): slot bounds, that the direct
  loads fill each tile once, that each MFMA operand read finds the rows and
  dims its lane supplies, and the bank-conflict-free reads; planted mistakes in
  a copy of the layout make that check fail;
- the same for the matrix-core decode's per-wavefront K and V buffers
  (decode_layout.h, through tests/host_build/decode_layout_check.cpp), at
  D = 128 and 64.

The host compiler is g++ (the C ABI layer includes only the HIP runtime's API
header), so no device code is built here."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "cross_layer_shared_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "host_build")
ROCM_INCLUDE = "/opt/rocm/include"

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INCLUDE),
                                reason="needs g++ and the HIP runtime headers")

COMMON = ["-std=c++20", "-g", "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE, "-I", os.path.join(ROOT, "include"),
          "-I", CSRC, "-I", HERE]


def _build_and_run(tmp_path, name, sources, flags, env=None):
    exe = str(tmp_path / name)
    cmd = ["g++", *COMMON, *flags, *sources, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, f"build failed:\n{r.stderr[-4000:]}"
    run = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert run.returncode == 0 and run.stdout.strip() == "ok", f"{run.stdout[-2000:]}\n{run.stderr[-4000:]}"


def test_abi_layer_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    _build_and_run(tmp_path, "abi_driver",
                   [os.path.join(CSRC, "yoco_api.cpp"), os.path.join(HERE, "launch_stubs.cpp"),
                    os.path.join(HERE, "abi_driver.cpp")],
                   ["-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"],
                   env)


def test_fastdiv_equals_division(tmp_path):
    # fastdiv.h is included by the kernels too; its host path needs only the HIP host macros
    _build_and_run(tmp_path, "fastdiv_check", [os.path.join(HERE, "fastdiv_check.cpp")],
                   ["-O2", "-include", "hip/hip_runtime.h"])


def test_prefill_lds_addresses(tmp_path):
    _build_and_run(tmp_path, "prefill_layout_check", [os.path.join(HERE, "prefill_layout_check.cpp")],
                   ["-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"])


# plausible slips in the layout, each of which the check must reject
LAYOUT_MUTATIONS = {
    "V rows loaded without their swizzle": ("return pos ^ (4 * (row & 3));", "return pos;"),
    "K operand chunk not swizzled by its row": ("16 * (q ^ (pk & 15))", "16 * q"),
    "K operand rows in plain order": ("pk = perm_key(j);", "pk = j;"),
    "transposing read without the row's chunk swizzle": ("* kRowB + 64 * r4 +", "* kRowB +"),
    "V^T write column in elements, not bytes": ("kVTRow + 2 * tr_first_key(wave, lane)", "kVTRow + tr_first_key(wave, lane)"),
    "PV operand keys of the wrong half": ("+ 16 * q + db * 32 * kVTRow", "+ 16 * (1 - q) + db * 32 * kVTRow"),
}


@pytest.mark.parametrize("name", sorted(LAYOUT_MUTATIONS))
def test_prefill_lds_address_check_rejects_planted_mistakes(tmp_path, name):
    old, new = LAYOUT_MUTATIONS[name]
    text = open(os.path.join(CSRC, "prefill_layout.h")).read()
    assert text.count(old) == 1, old
    (tmp_path / "prefill_layout.h").write_text(text.replace(old, new))
    src = tmp_path / "prefill_layout_check.cpp"     # next to the mutated header, which it then includes
    src.write_text(open(os.path.join(HERE, "prefill_layout_check.cpp")).read())
    exe = str(tmp_path / "check")
    r = subprocess.run(["g++", *COMMON, "-O1", str(src), "-o", exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert run.returncode != 0 and "FAIL" in run.stdout, f"{name}: not detected\n{run.stdout[-1000:]}"


def test_decode_lds_addresses(tmp_path):
    _build_and_run(tmp_path, "decode_layout_check", [os.path.join(HERE, "decode_layout_check.cpp")],
                   ["-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"])


DECODE_LAYOUT_MUTATIONS = {
    "K rows stored without their swizzle": ("8 * (load_chunk<D>(lane) ^ k_swizzle<D>(load_row<D>(i, lane)))",
                                            "8 * load_chunk<D>(lane)"),
    "score operand chunk not swizzled": ("8 * ((4 * j + (lane >> 4)) ^ k_swizzle<D>(k_row<D>(lane, bb)))",
                                         "8 * (4 * j + (lane >> 4))"),
    "score operand rows in plain order": ("return 8 * ((lane & 15) >> 2) + 4 * bb + (lane & 3);",
                                          "return (lane & 15) + 16 * bb;"),
    "transposing read of the wrong row quad": ("(8 * (lane >> 4) + 4 * h + ((lane & 15) >> 2))",
                                               "(8 * (lane >> 4) + 4 * (1 - h) + ((lane & 15) >> 2))"),
    "V rows without their pad": ("static constexpr int VPAD = D + 32;", "static constexpr int VPAD = D;"),
}


@pytest.mark.parametrize("name", sorted(DECODE_LAYOUT_MUTATIONS))
def test_decode_lds_address_check_rejects_planted_mistakes(tmp_path, name):
    old, new = DECODE_LAYOUT_MUTATIONS[name]
    text = open(os.path.join(CSRC, "decode_layout.h")).read()
    assert text.count(old) == 1, old
    (tmp_path / "decode_layout.h").write_text(text.replace(old, new))
    src = tmp_path / "decode_layout_check.cpp"
    src.write_text(open(os.path.join(HERE, "decode_layout_check.cpp")).read())
    exe = str(tmp_path / "check")
    r = subprocess.run(["g++", *COMMON, "-O1", str(src), "-o", exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert run.returncode != 0 and "FAIL" in run.stdout, f"{name}: not detected\n{run.stdout[-1000:]}"
