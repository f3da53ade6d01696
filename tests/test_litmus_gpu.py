"""Message-passing litmus test of the tile hand-off (publication: stores,
workgroup release, barrier, agent-scope release store of a flag;
consumption: relaxed agent-scope polls, hand-off acquire, operand DMA), in
one launch of 256 workgroups over many rounds, with producers and consumers
on different XCDs and consumers sharing an XCD with one of the two writers
of the lines they read.  Every wait is bounded by a host-set spin limit, so
the kernel always exits."""
import numpy as np
import pytest

from consumer_gemm_chain_amd import mlp_chain as mc

pytestmark = pytest.mark.gpu

ROUNDS = 64


def _litmus(half_lines, agent, rounds=ROUNDS):
    import torch
    data = torch.zeros(rounds << 20, dtype=torch.uint8, device="cuda")
    flags = torch.zeros(rounds * 256, dtype=torch.int32, device="cuda")
    res = torch.zeros(8, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    print(f"litmus rounds={rounds} half_lines={half_lines} agent={agent}", flush=True)
    mc.mlp_chain_debug_litmus(data.data_ptr(), data.numel(), flags.data_ptr(), flags.numel() * 4, res.data_ptr(),
                              rounds, half_lines, agent, 1 << 18, s)
    torch.cuda.synchronize()
    r = res.cpu().numpy().view(np.uint32)
    # every region was written in full by its two producers
    assert int(torch.count_nonzero(data.view(torch.int32))) == rounds * 128 * 2048
    return r


@pytest.mark.parametrize("half_lines,agent", [(False, False), (True, True)])
def test_handoff_litmus_as_the_chain_uses_it(half_lines, agent):
    """The two forms the chain uses: whole lines per producer with the
    workgroup-scope hand-off, and half lines (32-column producer tiles) with
    the agent-scope hand-off.  Not one word may be stale."""
    r = _litmus(half_lines, agent)
    assert r[6] == 0, "a wait exceeded the spin limit"
    assert r[0] == 0, f"{r[0]} stale words; first: round {r[1] - 1}, consumer {r[2]}, chunk {r[3]}, " \
                      f"read {r[4]:#x}, expected {r[5]:#x}"


def test_handoff_litmus_half_lines_with_workgroup_scope_is_reported():
    """Half lines from two XCDs with only the workgroup-scope hand-off (the
    form the chain no longer uses for such tiles): the count of stale words
    is reported, not asserted -- it shows what the L2 does with a line whose
    halves were written back by two XCDs."""
    r = _litmus(True, False)
    assert r[6] == 0
    print(f"half lines, workgroup-scope hand-off: {r[0]} stale words in {ROUNDS} rounds", flush=True)


def test_litmus_rejects_bad_sizes():
    import torch
    buf = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    lib = mc.load_library()
    p = buf.data_ptr()
    assert lib.mlp_chain_debug_litmus(p, buf.numel(), p, buf.numel(), p, 2, 1, 1, 0, None) == mc.MLP_EINVAL
    assert lib.mlp_chain_debug_litmus(None, 0, p, 1024, p, 1, 1, 1, 0, None) == mc.MLP_EINVAL
