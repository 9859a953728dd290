"""The entry point's smoke check runs as part of the GPU suite, so a change
that breaks it shows up with the other GPU tests."""
import pytest

pytestmark = pytest.mark.gpu


def test_smoke_entry_point():
    import __graft_entry__ as g
    g.smoke()
