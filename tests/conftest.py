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
