"""moe_weights_to_native on the GPU against the tests' numpy definition of
the native code order (tests/helpers.native_order): bit-exact."""
import sys

import numpy as np
import pytest
import torch

from tests.helpers import DEV, native_order

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wfmt,rows,cols", [
    (0, 32, 128),            # one strip pair, one chunk
    (0, 3 * 64, 384),        # three experts of 64 rows, three chunks
    (1, 32, 256),            # MXFP8: two parts per chunk
    (1, 2 * 48, 640),
    (0, 2048, 4096),         # one expert's w13 at the decode shapes (2I x H)
    (1, 4096, 1024),         # one expert's MXFP8 w2 (H x I)
])
def test_weights_to_native_bit_exact(wfmt, rows, cols):
    from mxfp4_routed_expert_top_amd import ops
    print("weights_to_native", wfmt, rows, cols, flush=True)
    sys.stdout.flush()
    rb = cols if wfmt == 1 else cols // 2
    g = torch.Generator().manual_seed(rows * 7 + cols + wfmt)
    src = torch.randint(0, 256, (rows, rb), generator=g, dtype=torch.uint8)
    got = ops.weights_to_native(src.to(DEV), wfmt)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), native_order(src.numpy(), 2 if wfmt == 1 else 1))


def test_weights_to_native_stacked_experts_and_empty():
    from mxfp4_routed_expert_top_amd import ops
    g = torch.Generator().manual_seed(5)
    src = torch.randint(0, 256, (4, 256, 128), generator=g, dtype=torch.uint8)   # [E', rows, H/2]
    got = ops.weights_to_native(src.to(DEV))
    torch.cuda.synchronize()
    for e in range(4):
        assert np.array_equal(got[e].cpu().numpy(), native_order(src[e].numpy(), 1))
    empty = torch.empty(0, 64, dtype=torch.uint8, device=DEV)
    assert ops.weights_to_native(empty).shape == (0, 64)
