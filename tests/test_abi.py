"""The C-ABI library on the CPU: it loads, exports every entry point the
header declares, its structs match the ctypes mirror, and host-side argument
checks reject bad calls before touching the GPU."""
import os
import re
import subprocess

import pytest

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


def _cfg(**kw):
    import synth
    c = dict(synth.config("tiny_flash_f32"))
    c.update(kw)
    return c


@pytest.mark.parametrize("bad,status", [
    (dict(P=6), 1),
    (dict(gate_hidden=32), 1),
    (dict(pool_heads=3), 1),
    (dict(C=62), 3),
    (dict(pool_layers=9), 1),
    (dict(ps_version=3), 1),
    (dict(ln_fold=2), 1),
    (dict(ln_fold=1), 2),  # the tiny workload is fp32: the fold needs bf16
])
def test_create_rejects_bad_config_on_host(bad, status):
    c = ivc.make_config(_cfg(**bad))
    w = ivc.ivc_weights()
    with pytest.raises(ivc.IvcError) as e:
        ivc.ivc_connector_create(c, w, 0)
    assert e.value.status == status


def test_create_rejects_bad_shuffle64_order_on_host():
    c = ivc.make_config(_cfg())
    c.shuffle64_order = 2
    with pytest.raises(ivc.IvcError) as e:
        ivc.ivc_connector_create(c, ivc.ivc_weights(), 0)
    assert e.value.status == 1


def test_create_rejects_missing_weights_on_host():
    c = ivc.make_config(_cfg())
    with pytest.raises(ivc.IvcError) as e:
        ivc.ivc_connector_create(c, ivc.ivc_weights(), 0)
    assert e.value.status == 1
    assert "missing" in ivc.ivc_last_error()


def test_entry_points_reject_bad_arguments_on_host():
    with pytest.raises(ivc.IvcError):
        ivc.ivc_tile_offsets(None, -1, None, None, 0)
    with pytest.raises(ivc.IvcError):
        ivc.ivc_pixel_shuffle(7, None, 1, 8, 64, 1, 2, None, 0)
    with pytest.raises(ivc.IvcError):
        ivc.ivc_pixel_shuffle(0, None, 1, 8, 64, 1, 3, None, 0)
    with pytest.raises(ivc.IvcError):
        ivc.ivc_pixel_shuffle(0, None, 1, 8, 64, 1, 2, None, 0, ps_version=3)
    with pytest.raises(ivc.IvcError):
        ivc.ivc_pixel_shuffle(0, None, 1, 8, 64, 1, 4, None, 0, shuffle64_order=2)
    with pytest.raises(ivc.IvcError) as e:
        ivc.ivc_pixel_shuffle(1, 18, 1, 8, 64, 1, 2, 34, 0)  # pointers not 16-byte aligned
    assert e.value.status == 3
    assert ivc.ivc_connector_workspace_bytes(None, 1, 1) == 0
    with pytest.raises(ivc.IvcError):
        ivc.ivc_connector_run(None, None, 1, None, None, None, 0, 0)
    assert ivc.ivc_status_string(4) == "workspace too small"
