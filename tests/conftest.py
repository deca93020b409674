import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; calls the HIP library")
    config.addinivalue_line("markers", "slow: CPU-heavy oracle work (tens of seconds)")


def pytest_collection_modifyitems(config, items):
    # GPU tests fail loudly (not skip) when run with -m gpu on a machine without
    # a GPU: a silent skip would hide a missing native path.
    pass


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library binding, on a machine that has the GPU."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but torch.cuda.is_available() is False")
    import io_aware_exact_fwd_amd as attn
    rc = attn.device_check(torch.cuda.current_device())
    assert rc == 0, attn.strerror(rc)
    return attn


def pytest_terminal_summary(terminalreporter):
    """Worst logged errors per test file (logged, not gated; see gpu_helpers)."""
    mod = sys.modules.get("gpu_helpers")
    log = getattr(mod, "ERROR_LOG", None) if mod else None
    if not log:
        return
    path = os.environ.get("ATTN_PARITY_LOG")
    if path:
        with open(path, "w") as f:
            for r in log:
                f.write(json.dumps(r) + "\n")
    tr = terminalreporter
    tr.section("parity errors (worst per file; abs = absolute, rel = / max|ref|)")
    tr.write_line(f"{'file':<24}{'kind':<5}{'n':>6}{'max':>11}{'mean':>11}{'vs rounded':>12}{'floor':>11}")
    groups = {}
    for r in log:
        groups.setdefault((r["test"].split("::")[0].split("/")[-1], r["kind"]), []).append(r)
    for (f, kind), rs in sorted(groups.items()):
        tr.write_line(f"{f:<24}{kind:<5}{len(rs):>6}" + "".join(
            f"{max(r[c] for r in rs):>{w}.3e}" for c, w in
            (("max", 11), ("mean", 11), ("max_vs_rounded_oracle", 12), ("rounding_floor", 11))))
