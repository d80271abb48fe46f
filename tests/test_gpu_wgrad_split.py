"""Weight gradients under imbalanced routing: experts holding many more rows than the others have
their row range split into parts whose FP32 partial tiles are summed in part order. Checked on a
Zipf(1.2)-biased routing where several experts split: the layer primitive and the stage calls agree
bit for bit (the split depends only on the per-expert row counts), repeated runs agree bit for bit,
the gradients match the oracle within the BF16 bounds, and the arrival counters in the workspace are
zero again after every call."""
import numpy as np
import pytest

import moe_inputs
from moe_inputs import MoeConfig

pytestmark = pytest.mark.gpu

harness = pytest.importorskip("harness")

CASES = [
    MoeConfig("zipf_small", T=4096, H=256, I=128, E=32, E_local=8, k=8, n_chunks=2, dtype="bf16", seed_base=700,
              zipf_s=1.2, n_empty=2, backward=True),
    MoeConfig("zipf_n3_h384", T=3000, H=384, I=320, E=64, E_local=16, e0=16, k=6, n_chunks=3, dtype="bf16",
              seed_base=710, zipf_s=1.2, n_empty=3, backward=True),
]


def _require_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import combine_moe_route_02_amd as mh
    mh.lib()


def _counters(run):
    import combine_moe_route_02_amd as mh
    ws = mh.workspace_bytes(run.desc)
    off = (max(ws["route_scratch"], ws["route_bwd_scratch"]) + 255) // 256 * 256
    return run.bufs["workspace"][off:off + ws["wgrad_zero_bytes"]].cpu().numpy()


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_split_weight_gradients(cfg):
    _require_gpu()
    print(f"[wgrad split] {cfg}", flush=True)
    a = harness.run_gpu(cfg)
    counts = a.bufs["offsets"].cpu().numpy()
    rows = (counts[:, 1:] - counts[:, :-1]).sum(axis=0)
    print("[wgrad split] rows per local expert", rows.tolist(), flush=True)
    assert rows.max() > 4 * max(1, np.median(rows))      # imbalanced enough that the plan splits
    assert np.all(_counters(a) == 0)
    ref = harness.run_oracle(a)
    print("[wgrad split]", harness.check_backward(a, ref), flush=True)
    b = harness.run_gpu(cfg, inp=a.inp, layer=False, two_streams=False)
    c = harness.run_gpu(cfg, inp=a.inp)
    for name in ("dw1", "dw2", "dx", "dwr"):
        np.testing.assert_array_equal(harness.bits_np(a.bufs[name]), harness.bits_np(b.bufs[name]), err_msg=name)
        np.testing.assert_array_equal(harness.bits_np(a.bufs[name]), harness.bits_np(c.bufs[name]), err_msg=name)
    assert np.all(_counters(b) == 0) and np.all(_counters(c) == 0)
