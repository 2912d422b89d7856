"""CPU checks of the test helpers themselves (no GPU)."""
import numpy as np
import torch

import tara_inputs as ti
from tara_testlib import run_oracle, run_oracle_all_heads


def test_oracle_over_worker_processes_matches_in_process():
    # the threaded path of the all-rows parity test gives exactly what
    # the in-process oracle gives, head by head
    lay = ti.make_layout(3, (2, 3), (2, 3), 2, 5, 7, mask=True)
    p = ti.Params(binding=True, gains=(1.25, 0.75))
    g = torch.Generator().manual_seed(11)
    q, k, v = (torch.randn((1, 3, lay.n, 16), generator=g).to(torch.bfloat16) for _ in range(3))
    o1, l1 = run_oracle(q, k, v, lay, p)
    o2, l2 = run_oracle_all_heads(q, k, v, lay, p, workers=3, row_block=37)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    o3, l3 = run_oracle_all_heads(q, k, v, lay, p, heads=[2, 0], row_block=50)
    assert np.array_equal(o3, o1[:, [2, 0]]) and np.array_equal(l3, l1[:, [2, 0]])
