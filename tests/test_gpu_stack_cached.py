"""GPU tests of the step-level replay/skip entry point (dit_stack_replay_cached):
computed steps are the captured graph's output bitwise, skipped steps are
the oracle's finite-difference prediction from the GPU's stored history."""
import numpy as np
import pytest

import dit_inputs as DI
from oracle import dit_oracle as O
from tests.parity import assert_parity, dev_bf16, host
from tests.test_gpu_block import STACK_TINY, _stack_inputs, cfg_of, rope_dev

pytestmark = pytest.mark.gpu


def _run(B, shape, blocks, x, tembs, rc, rs, fresh=None, t=None, chain=False):
    import torch
    cfg = cfg_of(B, shape, B.DIT_STACK_CHAIN if chain else 0)
    ws = B.alloc_workspace(B.stack_workspace_bytes(cfg, len(blocks)))
    n = tembs.shape[0]
    out = torch.empty(n, shape.seq_len, shape.dim, dtype=torch.bfloat16, device="cuda")
    st = B.Stack()
    if fresh is None:
        st.replay(cfg, [b.dev for b in blocks], dev_bf16(x), dev_bf16(tembs), rc, rs, out, ws)
    else:
        st.replay_cached(cfg, [b.dev for b in blocks], dev_bf16(x), dev_bf16(tembs), rc, rs, out, ws, fresh, t)
    torch.cuda.synchronize()
    st.close()
    return host(out)


@pytest.mark.parametrize("chain", [False, True])
def test_cached_replay(gpu_lib, chain):
    B = gpu_lib
    shape = STACK_TINY
    n_blocks, n_steps = 4, 7
    blocks, x, tembs = _stack_inputs(B, shape, n_blocks, n_steps)
    _, rc, rs = rope_dev(B, shape)
    print(f"cached replay chain={chain}", flush=True)
    fresh = [1, 1, 0, 1, 0, 0, 1]
    t = [1.0, 0.9, 0.75, 0.6, 0.4, 0.25, 0.1]
    got = _run(B, shape, blocks, x, tembs, rc, rs, fresh, t, chain)
    # all steps computed: the plain replay, bitwise
    allf = _run(B, shape, blocks, x, tembs, rc, rs, [1] * n_steps, None, chain)
    plain = _run(B, shape, blocks, x, tembs, rc, rs, None, None, chain)
    assert np.array_equal(allf, plain)
    hist = []
    for s in range(n_steps):
        if fresh[s]:
            if not chain or s < 2:
                assert np.array_equal(got[s], plain[s]), s
            else:
                # a computed step after a skipped one starts from the stored
                # prediction: one chained replay from out[s-1] reproduces it
                one = _run(B, shape, blocks, got[s - 1], tembs[s:s + 1], rc, rs, None, None, True)
                assert np.array_equal(got[s], one[0]), s
            hist.append(s)
        else:
            a, b = hist[-1], hist[-2]
            ref = O.extrapolate_step(got[a], got[b], t[s], t[a], t[b])
            assert_parity(got[s], ref, f"skipped step {s} chain={chain}")
            # fp32 arithmetic on bf16 history, one rounding to bf16: within
            # half an ulp of the prediction plus the fp32 rounding of its terms
            w = (t[s] - t[a]) / (t[a] - t[b])
            bound = 2.0 ** -8 * np.abs(ref) + 1e-6 * (1 + abs(w)) * (np.abs(got[a]) + np.abs(got[b]))
            assert np.all(np.abs(got[s] - ref) <= bound), s


def test_cached_replay_hold_with_one_computed_step(gpu_lib):
    B = gpu_lib
    shape = STACK_TINY
    blocks, x, tembs = _stack_inputs(B, shape, 2, 3)
    _, rc, rs = rope_dev(B, shape)
    got = _run(B, shape, blocks, x, tembs, rc, rs, [1, 0, 0], None)
    assert np.array_equal(got[1], got[0]) and np.array_equal(got[2], got[0])
    # uniform step times (t = None): step 2 = 2 out[1] - out[0]
    got = _run(B, shape, blocks, x, tembs, rc, rs, [1, 1, 0], None)
    ref = O.extrapolate_step(got[1], got[0], 2, 1, 0)
    assert_parity(got[2], ref, "skipped step, uniform times")
