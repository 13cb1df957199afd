import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; parity tests of the HIP path")
    config.addinivalue_line("markers", "slow: full-size cases (minutes of CPU work)")


@pytest.fixture(scope="session")
def orc():
    import oracle
    return oracle.get()


def _tally():
    gu = sys.modules.get("gpu_util")
    return (gu.SABOTAGE, gu.TALLY) if gu is not None else (False, None)


def pytest_terminal_summary(terminalreporter):
    sab, t = _tally()
    if t is not None and "sweep" in t:
        f, c, ctrl = t["sweep"]
        terminalreporter.write_line(f"sabotage sweep: {f} of {c} packed-weight checks failed on corrupted bytes; "
                                    f"dense fp16 control {'passed' if ctrl else 'FAILED'}")
    if t is None or not (sab or t["checks"]):
        return
    line = (f"packed-weight checks: {t['checks']}, failed: {t['failed']}; controls: {t['controls']}, "
            f"passed: {t['controls_passed']}")
    if sab:
        line = "SABOTAGE (QGEMV_SABOTAGE=1) " + line
        if t["unfailed"]:
            line += "; checks that did not see the corruption: " + ", ".join(t["unfailed"][:20])
    terminalreporter.write_line(line)


def pytest_sessionfinish(session, exitstatus):
    sab, t = _tally()
    if sab and t is not None and (t["failed"] != t["checks"] or t["controls_passed"] != t["controls"]):
        session.exitstatus = 1
