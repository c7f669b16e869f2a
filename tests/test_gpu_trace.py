"""The traced indexer entry point (per-workgroup CU ids and timestamps of the
causal stream kernel) returns the untraced call's indices bit for bit under
every tile schedule, and its records are complete and consistent: one per
workgroup of the persistent grid, ends after starts, every query tile
accounted for once."""
import numpy as np
import pytest
import torch

import indexer_top_sparse_02_amd as sia
import workloads as W
from _paths import gpu_topk

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("sched", [0, 1, 2])
def test_traced_stream_kernel_matches_and_records(sched):
    s = W.spec("prefill_16k", ctx_lo=3000, ctx_hi=3000, topk=256, idx_fp8=True)
    wl = W.make(s, device="cuda")
    ref, _ = gpu_topk(wl, sched=sched)
    n_tiles = (wl.num_q + 3) // 4
    trace = torch.zeros((n_tiles, 4), dtype=torch.int64, device="cuda")
    got = sia.sparse_indexer_topk_traced(wl.page_table, wl.seq_lens, wl.idx_k, wl.idx_scale, wl.q_seq,
                                         wl.q_pos, wl.q_idx, wl.w, s.topk, trace, group=wl.num_q,
                                         sched=sched)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    t = trace.cpu().numpy()
    used = t[t[:, 2] != 0]
    assert len(used) >= 1
    assert np.all(used[:, 2] >= used[:, 1])
    # every query tile ran exactly once over all workgroups, which are
    # persistent (at most two per CU, each pulling tiles from a counter)
    assert int(used[:, 3].sum()) == n_tiles
    assert len(used) <= 2 * torch.cuda.get_device_properties(0).multi_processor_count
