import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


# With COSA_OSK_HEALTH_CHECK set to a file path, every prefill call made through the runner
# helpers is followed by a device synchronisation and a read of the workspace health word,
# which must be 0, and appends one line to that file.  The bounds-checked library counts
# index-invariant violations in the health word, so a run of the parity tests against it
# (tests/test_gpu_checked.py) fails on the first call that breaks one.
@pytest.fixture(autouse=True)
def _health_checked_prefill(monkeypatch):
    record = os.environ.get("COSA_OSK_HEALTH_CHECK")
    if not record:
        yield
        return
    from block_sparse_long_osk_amd import runner
    plain = runner.prefill

    def checked(db, order_mask, mask_len, delta, *args, **kw):
        import torch
        width = int(order_mask.shape[2])
        if kw.get("workspace") is None:
            kw["workspace"] = runner.workspace_for(db, width)
        outs = plain(db, order_mask, mask_len, delta, *args, **kw)
        if db.total_qblocks == 0:  # nothing launched: the workspace is not written
            return outs
        torch.cuda.synchronize()
        bad = runner.abort_count(db, kw["workspace"], width)
        assert bad == 0, f"the checked kernels counted {bad} index-invariant violations"
        with open(record, "a") as f:
            f.write(f"{db.total_qblocks} {width} 0\n")
        return outs

    monkeypatch.setattr(runner, "prefill", checked)
    yield
