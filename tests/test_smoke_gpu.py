"""The package's smoke check (one small layer forward on cuda:0 against the
oracle) passes as a GPU test too."""
import pytest

pytestmark = pytest.mark.gpu


def test_smoke_entry_point():
    import __graft_entry__
    __graft_entry__.smoke()
