"""The smoke check's reduced workloads build valid routings and inputs (CPU);
smoke() itself needs the GPU."""
import numpy as np

import __graft_entry__ as entry
import workloads as W


def test_smoke_workloads_build():
    for name in entry.SMOKE_SHAPES:
        w = entry.smoke_workload(name)
        r = W.routing(w)
        assert r.total_rows > 0 and (r.counts > 0).any()
        x = W.activations(w, r)
        assert tuple(x.shape) == (r.total_rows, w.K)
        assert np.all(np.diff(r.row_offsets.astype(np.int64)) >= 0)
