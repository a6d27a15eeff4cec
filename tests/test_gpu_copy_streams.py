"""The measurement entry point sim_copy_streams (k independent streaming
copies in one launch, the one-shot's access pattern without its
arithmetic): every destination equals its source byte for byte, for every
k, ragged vector counts and forced grid sizes; argument errors enqueue
nothing."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def lib():
    import all_reduce_reduction_amd as sim
    sim.sim_init(0, 16, 0)
    yield sim


def _bufs(k, nbytes, seed):
    import torch
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    src = [torch.randint(-2 ** 31, 2 ** 31 - 1, (max(nbytes // 4, 1),), generator=g, dtype=torch.int32).cuda()
           for _ in range(k)]
    dst = [torch.full((max(nbytes // 4, 1),), -0x5A5A5A5B, dtype=torch.int32, device="cuda") for _ in range(k)]
    return src, dst


@pytest.mark.parametrize("k", [1, 2, 3, 4, 7, 8, 16])
@pytest.mark.parametrize("nbytes,wg", [(16, 0), (16 * 255, 0), (16 * 257, 0), (16 * (3 * 256 + 17), 2),
                                       (1 << 20, 0), (1 << 20, 7), ((1 << 24) + 48, 1000)])
def test_copies_are_exact(lib, k, nbytes, wg):
    import torch
    from tests.gpu_util import ptrs, stream
    src, dst = _bufs(k, nbytes, k * 1000 + nbytes % 997)
    assert lib.sim_copy_streams(ptrs(src), ptrs(dst), k, nbytes, wg, stream()) == 0
    torch.cuda.synchronize()
    w = nbytes // 4
    for q in range(k):
        assert torch.equal(dst[q][:w], src[q][:w]), (k, nbytes, wg, q)
        assert (dst[q][w:] == -0x5A5A5A5B).all()  # nothing past the end


def test_argument_errors_enqueue_nothing(lib):
    import torch
    from tests.gpu_util import ptrs, stream
    src, dst = _bufs(2, 4096, 1)
    s, d = ptrs(src), ptrs(dst)
    cases = [
        (s, d, 0, 4096, 0, -1),                  # k < 1
        (s, d, 17, 4096, 0, -1),                 # k > SIM_MAX_RANKS
        (s, d, 2, 4095, 0, -1),                  # not a multiple of 16
        (s, d, 2, 4096, -1, -1),                 # negative grid
        ([s[0], 0], d, 2, 4096, 0, -1),          # NULL source
        (s, [d[0] + 4, d[1]], 2, 4080, 0, -3),   # misaligned destination
        (s, [d[0], d[0] + 1024], 2, 2048, 0, -4),  # destinations overlap
        (s, [s[1], d[1]], 2, 4096, 0, -4),       # destination overlaps a source
    ]
    for a in cases:
        assert lib.sim_copy_streams(a[0], a[1], a[2], a[3], a[4], stream()) == a[5], a[2:]
    assert lib.sim_copy_streams(s, d, 2, 0, 0, stream()) == 0   # zero bytes: no-op
    torch.cuda.synchronize()
    assert all((t == -0x5A5A5A5B).all() for t in dst)
