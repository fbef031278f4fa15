"""GPU parity of the compensator update run beside the next matmul.

The PhantomByte article ("The cancellation rule") places the two-timescale
compensator's update off the critical path, next to the following matrix
multiplication, and says this leaves the computed values as they were.  Here
echo_compensate runs on a second HIP stream while a bf16 matmul (the shape of
a Llama-3-8B gate/up projection at TP = 4, hipBLASLt through torch) runs on the
main stream, joined by events.  Over three consecutive updates that carry the
slow memory, the compensation and slow memory match the oracle's update bit
for bit, and the matmul's result is bit-identical to the same matmul run
alone."""
import numpy as np
import pytest
import torch

import oracle
from _helpers import DEV, assert_bits_equal, dev_f32, host_f32, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def echo():
    from error_feedback_quant_amd import echo as e
    assert torch.cuda.is_available()
    return e


@pytest.mark.parametrize("alpha, beta", [(0.5, 0.25), (1.0, 0.0)])
def test_update_beside_matmul_matches_oracle(echo, alpha, beta):
    n = (1 << 22) + 12                       # several blocks and a scalar tail
    rng = np.random.default_rng(4242)
    M, K, N = 4096, 4096, 7168
    g = torch.Generator(device="cpu").manual_seed(17)
    a = torch.randn(M, K, generator=g).to(torch.bfloat16).to(DEV).contiguous()
    w = (torch.randn(N, K, generator=g) * K ** -0.5).to(torch.bfloat16).to(DEV).contiguous()
    wt = w.t().contiguous()                  # [K, N], contiguous right operand
    alone = torch.matmul(a, wt)
    torch.cuda.synchronize()
    alone_h = alone.view(torch.int16).cpu().numpy()

    comp_h = np.zeros(n, np.float32)
    slow_h = (rng.standard_normal(n) * 1e-3).astype(np.float32) if beta > 0 else None
    comp_d = dev_f32(comp_h)
    slow_d = dev_f32(slow_h) if beta > 0 else None
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    for call in range(3):
        e_h = (rng.standard_normal(n) * 10.0 ** rng.uniform(-4, -1)).astype(np.float32)
        e_d = dev_f32(e_h)
        say("update beside matmul", alpha, beta, "call", call)
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event()
        ev0.record(main)
        side.wait_event(ev0)
        z = torch.matmul(a, wt)              # main stream
        echo.echo_compensate(e_d, comp_d, slow_d, n, alpha, beta, stream=side)
        ev1 = torch.cuda.Event()
        ev1.record(side)
        main.wait_event(ev1)
        torch.cuda.synchronize()
        oracle.compensate(e_h, comp_h, slow_h, n, alpha, beta)
        assert_bits_equal(host_f32(comp_d), comp_h, f"comp, call {call}")
        if beta > 0:
            assert_bits_equal(host_f32(slow_d), slow_h, f"slow, call {call}")
        assert_bits_equal(z.view(torch.int16).cpu().numpy(), alone_h, f"matmul beside the update, call {call}")
