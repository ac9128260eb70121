"""fi_set_block_weights_static, the weight upload for callers that cannot
allocate device memory: through the C-ABI it must give exactly what
fi_set_block_weights gives.  Two calls in a row share the library's static
staging array, the second with a smaller input (its array still holds the
first call's values past the second's end); host and device sources; and a
block wider than the array holds is refused."""
import numpy as np
import pytest
import torch

from long_convolution_sequence_amd import fi, workloads
from tests._parity import say

pytestmark = pytest.mark.gpu


def _outputs(w, bits, static, on_device, steps):
    h = workloads.filters(w)
    x1 = torch.from_numpy(workloads.x_first(w)).cuda()
    with fi.Context(torch.from_numpy(h).cuda(), w.B, map=fi.MAP_HYENA, tau_split=4) as ctx:
        args = [bits[k] for k in ("W", "W1", "W2")]
        if on_device:
            args = [torch.from_numpy(a.view(np.int16)).cuda() for a in args]
        (ctx.set_block_weights_static if static else ctx.set_block_weights)(*args)
        ctx.set_input(x1)
        return ctx.generate(steps).cpu().numpy()


@pytest.mark.parametrize("on_device", [False, True])
def test_static_weight_upload_equals_allocating_one(on_device):
    steps = 96
    for M, B, D in ((3, 2, 64), (2, 1, 32)):              # second call smaller than the first
        w = workloads.custom(M=M, B=B, D=D, L=256, decay=32.0, scale=0.5, seed=61 + D, block="hyena")
        say(f"case static weight upload M={M} B={B} D={D} on_device={on_device}")
        bits = workloads.hyena_weights(w)
        y_static = _outputs(w, bits, True, on_device, steps)
        y_alloc = _outputs(w, bits, False, on_device, steps)
        assert np.isfinite(y_static).all() and np.abs(y_static).max() > 0
        assert np.array_equal(y_static, y_alloc)


def test_blocks_wider_than_the_static_scratch_are_refused():
    """The block mode takes D <= 768, which is also what the static staging
    array holds (4 * 768 * 768 16-bit values): a wider block is refused when the
    context is made, before any upload could need more."""
    w = workloads.custom(M=1, B=1, D=776, L=8, decay=4.0, seed=5, block="hyena")
    h = workloads.filters(w)
    say("case block wider than 768 refused")
    with pytest.raises(fi.FiError) as e:
        fi.Context(torch.from_numpy(h).cuda(), w.B, map=fi.MAP_HYENA, tau_split=2)
    assert e.value.status == fi.FI_EINVAL
