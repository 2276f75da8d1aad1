"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, host only): every entry point runs on small inputs with edge lengths,
element masks and every variant, and the run must report nothing."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE = os.path.join(os.path.dirname(HERE), "oracle")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_is_clean_under_asan_and_ubsan(tmp_path):
    src = os.path.join(ORACLE, "oracle.c")
    driver = os.path.join(ORACLE, "sanitize_driver.c")
    exe = str(tmp_path / "oracle_sanitized")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-g", "-O1", "-std=c11"]
    objs = []
    for real, sfx, extra in (("double", "_f64", ["-DORACLE_WITH_BLOCKMASK"]), ("float", "_f32", [])):
        obj = str(tmp_path / f"oracle{sfx}.o")
        subprocess.check_call(["gcc", *san, f"-DREAL={real}", f"-DSFX={sfx}", *extra, "-c", src,
                               "-o", obj])
        objs.append(obj)
    subprocess.check_call(["gcc", *san, driver, *objs, "-lm", "-o", exe])
    # verify_asan_link_order=0: the environment may preload a library of its
    # own ahead of the sanitizer runtime.
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0, res.stderr[-4000:]
    assert res.stdout.startswith("ok"), res.stdout
    assert "runtime error" not in res.stderr, res.stderr[-4000:]
