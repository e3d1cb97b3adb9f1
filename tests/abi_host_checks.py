"""Host-side argument checks of the C ABI, callable without a GPU: every call
here must be rejected on the host with the stated status, before anything is
enqueued.  test_abi.py runs them in-process against libivc.so, and again in a
child process against the host-sanitized build (AddressSanitizer +
UndefinedBehaviorSanitizer), where any memory or UB error ends the child with
a non-zero status.

    IVC_LIBRARY=<lib> python tests/abi_host_checks.py
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from vlm_visual_token_amd import ivc  # noqa: E402

BAD_CONFIGS = [
    (dict(P=6), 1),
    (dict(gate_hidden=32), 1),
    (dict(pool_heads=3), 1),
    (dict(C=62), 3),
    (dict(pool_layers=9), 1),
    (dict(ps_version=3), 1),
    (dict(ln_fold=2), 1),
    (dict(ln_fold=1), 2),  # the tiny workload is fp32: the fold needs bf16
]


def cfg(**kw):
    import synth
    c = dict(synth.config("tiny_flash_f32"))
    c.update(kw)
    return c


def expect_status(fn, status=None):
    try:
        fn()
    except ivc.IvcError as e:
        assert status is None or e.status == status, (e.status, status, str(e))
        return e
    raise AssertionError("call was not rejected")


def check_bad_config(bad, status):
    c = ivc.make_config(cfg(**bad))
    expect_status(lambda: ivc.ivc_connector_create(c, ivc.ivc_weights(), 0), status)


def check_bad_shuffle64_order():
    c = ivc.make_config(cfg())
    c.shuffle64_order = 2
    expect_status(lambda: ivc.ivc_connector_create(c, ivc.ivc_weights(), 0), 1)


def check_missing_weights():
    c = ivc.make_config(cfg())
    expect_status(lambda: ivc.ivc_connector_create(c, ivc.ivc_weights(), 0), 1)
    assert "missing" in ivc.ivc_last_error()


def check_entry_points():
    expect_status(lambda: ivc.ivc_tile_offsets(None, -1, None, None, 0))
    expect_status(lambda: ivc.ivc_pixel_shuffle(7, None, 1, 8, 64, 1, 2, None, 0))
    expect_status(lambda: ivc.ivc_pixel_shuffle(0, None, 1, 8, 64, 1, 3, None, 0))
    expect_status(lambda: ivc.ivc_pixel_shuffle(0, None, 1, 8, 64, 1, 2, None, 0, ps_version=3))
    expect_status(lambda: ivc.ivc_pixel_shuffle(0, None, 1, 8, 64, 1, 4, None, 0,
                                                shuffle64_order=2))
    # pointers not 16-byte aligned
    expect_status(lambda: ivc.ivc_pixel_shuffle(1, 18, 1, 8, 64, 1, 2, 34, 0), 3)
    assert ivc.ivc_connector_workspace_bytes(None, 1, 1) == 0
    expect_status(lambda: ivc.ivc_connector_run(None, None, 1, None, None, None, 0, 0))
    expect_status(lambda: ivc.ivc_connector_compact_noalloc(None, None, None, 1, 0, None, None,
                                                            None, 1, None, None, None, None, None,
                                                            None, 0), 1)
    assert ivc.ivc_status_string(4) == "workspace too small"
    for s in range(-1, 9):
        assert isinstance(ivc.ivc_status_string(s), str)


def run_all():
    for bad, status in BAD_CONFIGS:
        check_bad_config(bad, status)
    check_bad_shuffle64_order()
    check_missing_weights()
    check_entry_points()


if __name__ == "__main__":
    ivc.load()
    run_all()
    print(f"host checks ok ({ivc.LIB_PATH})")
