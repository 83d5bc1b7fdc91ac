"""__graft_entry__.smoke() runs on the GPU (one small append + decode against
the oracle), so a change that breaks it fails the GPU suite as well."""
import pytest

pytestmark = pytest.mark.gpu


def test_smoke_runs():
    import __graft_entry__ as g
    g.smoke()
