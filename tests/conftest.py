import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "error_word_expected: the test sets a workspace error "
                                       "word on purpose (and checks it itself)")


def _gpu_visible() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


@pytest.fixture(autouse=True)
def _workspace_error_words_stay_zero(request):
    """After every GPU test, every workspace the binding's helpers created during the test
    (directly, or inside a call that was given none) must hold a zero error word: no expert
    id out of range and no wait between workgroups that gave up."""
    if "gpu" not in request.keywords or not _gpu_visible():
        yield
        return
    import torch
    from dequant_gemv_amd import binding as B
    made, orig = [], {}
    for name in ("moe_workspace", "gemv_workspace"):
        f = getattr(B, name)
        orig[name] = f

        def wrapped(*a, _f=f, **k):
            t = _f(*a, **k)
            if t is not None:
                made.append(t)
            return t
        setattr(B, name, wrapped)
    try:
        yield
    finally:
        for name, f in orig.items():
            setattr(B, name, f)
    if "error_word_expected" in request.keywords:
        return
    torch.cuda.synchronize()
    for t in made:
        word = int(t[:4].view(torch.int32).item())
        assert word == 0, f"workspace error word {word:#x} after the test"


def pytest_collection_modifyitems(config, items):
    # GPU tests stay in the suite on a CPU-only machine but are skipped there.
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)
