"""The achievable-rate probes of libyoco_ceiling.so touch every byte they are
timed on, so no ceiling is inflated by skipped work:

- the four-reads-two-writes probe writes e = a + b and f = c + d (32-bit
  integer adds) over the whole buffers, for every positions-per-thread and
  thread count the bench sweeps, on a size that is not a multiple of a
  workgroup's share;
- each read probe (threads striding over a workgroup's range, or wavefronts
  taking blocks) loads every 16-byte vector: with one key word planted in an
  otherwise zero buffer, the thread that loads it holds the key as its XOR
  and writes the sink, wherever the key sits (first, last, middle, seeded);
- the matrix-core probe runs on any operand pool and leaves the sink alone."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

SINK_KEY = 0x9E3779B9


@pytest.fixture(scope="module")
def C():
    from cross_layer_shared_amd import ceiling
    ceiling.load_ceiling_library()
    return ceiling


@pytest.mark.parametrize("threads,u", [(256, 1), (512, 1), (1024, 1), (256, 2), (512, 2), (256, 4)])
def test_read4_write2_writes_every_sum(C, threads, u):
    n = 4 * 300_007                        # int32 words: 300,007 16-byte vectors
    g = torch.Generator(device="cuda").manual_seed(threads * 10 + u)
    a, b, c, d = (torch.randint(-2**30, 2**30, (n,), dtype=torch.int32, device="cuda", generator=g) for _ in range(4))
    e = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    f = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    C.yoco_ceiling_read4_write2(a, b, c, d, e, f, threads=threads, positions_per_thread=u)
    torch.cuda.synchronize()
    assert torch.equal(e, a + b) and torch.equal(f, c + d)


def _planted(n_vec, at):
    buf = torch.zeros(4 * n_vec, dtype=torch.int32, device="cuda")
    buf[4 * at + 2] = np.array(SINK_KEY, dtype=np.uint32).view(np.int32).item()
    return buf


@pytest.mark.parametrize("mode,wg,threads,u", [("stride", 256, 512, 4), ("stride", 256, 512, 16), ("stride", 1024, 256, 8),
                                                ("stride", 0, 512, 8), ("blocks", 256, 512, 4), ("blocks", 1024, 256, 8),
                                                ("blocks", 2048, 256, 8)])
def test_read_probes_load_every_vector(C, mode, wg, threads, u):
    n_vec = 1_000_003
    rng = np.random.default_rng(wg + threads + u)
    for at in (0, n_vec - 1, n_vec // 2, int(rng.integers(n_vec))):
        src = _planted(n_vec, at)
        sink = torch.zeros(4, dtype=torch.int32, device="cuda")
        if mode == "stride":
            C.yoco_ceiling_read(src, sink, workgroups=wg, threads=threads, loads_per_thread=u)
        else:
            C.yoco_ceiling_read_blocks(src, sink, workgroups=wg, threads=threads, loads_per_thread=u)
        torch.cuda.synchronize()
        got = int(np.array(sink[0].item(), dtype=np.int32).view(np.uint32))
        assert got == SINK_KEY, f"{mode} {wg}x{threads}x{u}: vector {at} of {n_vec} was not read"


def test_mfma_probe_runs_and_leaves_the_sink(C):
    sink = torch.zeros(4, dtype=torch.float32, device="cuda")
    for pool in (torch.randn(1 << 16, device="cuda").to(torch.bfloat16), torch.zeros(256, dtype=torch.bfloat16, device="cuda")):
        C.yoco_ceiling_mfma_bf16(pool, sink, workgroups=8, iters=4)
    torch.cuda.synchronize()
    assert torch.all(sink == 0)
    assert C.mfma_flop(256, 16384) == 256 * 8 * 16384 * 16 * 32768
