import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


import pytest  # noqa: E402


@pytest.fixture(autouse=True)
def _checked_cache_writes(request, monkeypatch):
    """Every cache write a GPU test makes goes through the slot validation
    pass first (unique, in-range slots: the write's precondition).  CPU
    tests call the binding with deliberately bad arguments and are left
    alone."""
    if request.node.get_closest_marker("gpu") is None:
        yield
        return
    import mla_paged_decode_concat_amd as M
    from helpers import check_slots
    real = M.cache_write

    def checked(kv_c, k_pe, kv_cache, slot_mapping, *args, **kwargs):
        import torch
        if not torch.cuda.is_current_stream_capturing():   # a graph capture cannot read the slots back
            check_slots(slot_mapping, kv_cache.shape[0], kv_cache.shape[1])
        return real(kv_c, k_pe, kv_cache, slot_mapping, *args, **kwargs)

    monkeypatch.setattr(M, "cache_write", checked)
    yield
