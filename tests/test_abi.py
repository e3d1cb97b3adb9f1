"""The C-ABI library on the CPU: it loads, exports every entry point the
header declares, its structs match the ctypes mirror, and host-side argument
checks reject bad calls before touching the GPU."""
import os
import re
import subprocess
import sys

import pytest

from tests import abi_host_checks as H
from vlm_visual_token_amd import ivc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ivc.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ivc_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = ivc.load()
    names = _declared()
    assert "ivc_connector_create" in names and "ivc_connector_compact" in names
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(ivc.exported_symbols()) == names


def test_struct_layout_matches_header(tmp_path):
    import ctypes
    prog = tmp_path / "lay.c"
    fields_c = [f for f, _ in ivc.ivc_config._fields_]
    fields_w = [f for f, _ in ivc.ivc_weights._fields_]
    lines = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{HEADER}"', 'int main(void){',
             'printf("%zu %zu\\n", sizeof(ivc_config), sizeof(ivc_weights));']
    lines += [f'printf("%zu\\n", offsetof(ivc_config, {f}));' for f in fields_c]
    lines += [f'printf("%zu\\n", offsetof(ivc_weights, {f}));' for f in fields_w]
    lines += ["return 0;}"]
    prog.write_text("\n".join(lines))
    exe = tmp_path / "lay"
    subprocess.check_call(["gcc", "-std=c99", "-o", str(exe), str(prog)])
    out = subprocess.check_output([str(exe)]).decode().split()
    assert int(out[0]) == ctypes.sizeof(ivc.ivc_config)
    assert int(out[1]) == ctypes.sizeof(ivc.ivc_weights)
    offs = [int(v) for v in out[2:]]
    exp = [getattr(ivc.ivc_config, f).offset for f in fields_c] + \
          [getattr(ivc.ivc_weights, f).offset for f in fields_w]
    assert offs == exp


@pytest.mark.parametrize("bad,status", H.BAD_CONFIGS)
def test_create_rejects_bad_config_on_host(bad, status):
    H.check_bad_config(bad, status)


def test_create_rejects_bad_shuffle64_order_on_host():
    H.check_bad_shuffle64_order()


def test_create_rejects_missing_weights_on_host():
    H.check_missing_weights()


def test_entry_points_reject_bad_arguments_on_host():
    H.check_entry_points()


# The same host checks in a child process against the library built with
# AddressSanitizer and UndefinedBehaviorSanitizer on its host code, and the
# sanitized index-math self-test.  CPU only: no GPU code runs.
@pytest.mark.slow
def test_host_checks_under_address_and_ub_sanitizers():
    from vlm_visual_token_amd import build
    san = build.build_sanitized()
    r = subprocess.run([san["selftest"]], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, IVC_LIBRARY=san["lib"], LD_PRELOAD=san["asan_runtime"],
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "abi_host_checks.py")],
                       capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "host checks ok" in r.stdout and san["lib"] in r.stdout


def test_trace_log_names_entry_calls():
    script = os.path.join(ROOT, "tests", "abi_host_checks.py")
    on = subprocess.run([sys.executable, script], capture_output=True, text=True, timeout=300,
                        env=dict(os.environ, IVC_TRACE="1"))
    assert on.returncode == 0, on.stderr[-2000:]
    lines = [ln for ln in on.stderr.splitlines() if ln.startswith("[ivc] ")]
    assert any(ln.startswith("[ivc] create dtype=0 C=64 P=6") for ln in lines)
    assert any(ln.startswith("[ivc] pixel_shuffle dtype=7") for ln in lines)
    assert any(ln.startswith("[ivc] tile_offsets B=-1") for ln in lines)
    off = subprocess.run([sys.executable, script], capture_output=True, text=True, timeout=300,
                         env=dict(os.environ, IVC_TRACE="0"))
    assert off.returncode == 0 and "[ivc]" not in off.stderr
