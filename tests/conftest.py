import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_sessionfinish(session, exitstatus):
    """With QLORA_LIBRARY=checked every GPU test ran through the
    bounds-checked build: the run fails if any access fell outside its
    buffer."""
    if os.environ.get("QLORA_LIBRARY") != "checked":
        return
    import torch
    if not torch.cuda.is_available():
        return
    from bit_nf4_quantized_double_amd import qlora
    n = qlora.debug_oob_count(reset=True)
    print(f"\nbounds-checked build: {n} out-of-range accesses")
    if n:
        session.exitstatus = 1
