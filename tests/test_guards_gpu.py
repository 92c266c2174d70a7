"""The guard bytes the parity tests wrap around GPU outputs: a write just
past either end of the tensor (made here on purpose with a torch copy inside
the same allocation) is detected; an untouched buffer passes."""
import numpy as np
import pytest

from common import GUARD_BYTES, Guarded

pytestmark = pytest.mark.gpu


def test_guards_detect_writes_past_either_end():
    g = Guarded(np.zeros((3, 5), np.uint16))
    g.check("clean")
    assert g.view().data_ptr() % 256 == 0
    g.buf[GUARD_BYTES + g.nbytes] = 0
    with pytest.raises(AssertionError):
        g.check("tail")
    g = Guarded(np.zeros(7, np.float32))
    g.buf[GUARD_BYTES - 1] = 0
    with pytest.raises(AssertionError):
        g.check("head")
