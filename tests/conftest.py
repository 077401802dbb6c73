import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD GPU (MI355X, gfx950) and the built HIP library")
    # Full-size parity runs the fp64 oracle in worker processes.  Their
    # fork server starts here, before this process touches the GPU, so no
    # worker is ever forked from a process that holds a GPU context.
    import multiprocessing
    import multiprocessing.forkserver as fs
    multiprocessing.get_context("forkserver").set_forkserver_preload(
        ["numpy", "oracle.wise_oracle", "block_sparse_paged_split_amd.synth"])
    fs.ensure_running()


def _gpu_present() -> bool:
    try:
        import torch
        return torch.cuda.is_available() and torch.cuda.device_count() > 0
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if _gpu_present():
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Selection ambiguity classes over every GPU-vs-oracle comparison of the
    session: units compared, units in class A (cut within 1e-6 of eta) and
    class B (tied boundary masses), and support mismatches, each of which
    was exactly a moved cut or a tied swap.  Also written as JSON to the path
    in WISE_PARITY_RECORD, when set."""
    mod = sys.modules.get("parity")
    recs = getattr(mod, "RECORDS", None) if mod else None
    if not recs:
        return
    tot = {k: sum(r[k] for r in recs) for k in ("units", "near_eta", "near_tie", "mismatch",
                                                 "excused_a", "excused_b")}
    tr = terminalreporter
    tr.write_sep("-", "selection ambiguity classes (GPU vs oracle)")
    tr.write_line(f"{len(recs)} calls, {tot['units']} units compared: class A {tot['near_eta']}, "
                  f"class B {tot['near_tie']}; support mismatches {tot['mismatch']} "
                  f"(moved cut {tot['excused_a']}, tied swap {tot['excused_b']})")
    path = os.environ.get("WISE_PARITY_RECORD")
    if path:
        import json
        os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
        with open(path, "w") as f:
            json.dump({"totals": tot, "calls": recs}, f, indent=1)
