import importlib.util
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def _load_file(name, path):
    spec = importlib.util.spec_from_file_location(name, path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    # The libraries are built ahead of time; a fresh checkout without them
    # (they are not committed) gets them built once here.  The build module is
    # loaded by path: importing the package itself needs the built library.
    lib = os.path.join(ROOT, "sparse_attention_token_02_amd", "libdsa_indexer.so")
    if not os.path.exists(lib):
        _load_file("_dsa_build", os.path.join(ROOT, "sparse_attention_token_02_amd", "build.py")).build()
    syn = os.path.join(ROOT, "synth", "libdsa_synth.so")
    if not os.path.exists(syn):
        import synth.gpu as sg
        sg.build()


# ---- parity report: rows compared, rows the rounding floor decided, and the
# worst score errors, per test (printed in the terminal summary)
_PARITY_REPORT = []


def pytest_runtest_call(item):
    try:
        from tests import parity
    except Exception:
        return
    parity.reset_stats()


def pytest_runtest_teardown(item, nextitem):
    try:
        from tests import parity
    except Exception:
        return
    st = dict(parity.STATS)
    if st["rows"]:
        _PARITY_REPORT.append((item.nodeid, st, parity.take_floor_rows()))


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    if not _PARITY_REPORT:
        return
    tr = terminalreporter
    tr.section("parity: rows checked / floor-decided rows / worst score error")
    tot_rows = tot_floor = 0
    for nodeid, st, floor in _PARITY_REPORT:
        tot_rows += st["rows"]
        tot_floor += st["floor_rows"]
        line = (f"{nodeid}: rows {st['rows']}, floor-decided {st['floor_rows']}, "
                f"max |err|/|o| {st['max_err_rel_o']:.2e} (|o| >= 0.1 A), max |err|/A {st['max_err_rel_A']:.2e}")
        if floor:
            line += " | floor rows (id, max |o-tau|/|tau|): " + ", ".join(f"({r}, {d:.2e})" for r, d in floor[:8])
        tr.write_line(line)
    tr.write_line(f"total: {tot_rows} rows, {tot_floor} floor-decided")
