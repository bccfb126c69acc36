"""GPU parity of the DDP communication hook at world size 1 (one process, NCCL on the one
GPU): every bucket DDP hands to the hook, over three training iterations, is checked bit
for bit against the oracle's EF step (carrying the oracle's residual per bucket) followed
by the oracle's receive (average of W = 1 decoded payloads into +0.0), with the hook's
work on its side stream and on DDP's own stream."""
import socket

import numpy as np
import pytest

import oracle
from gc_testlib import assert_bits_equal

pytestmark = pytest.mark.gpu

F32 = np.float32


@pytest.fixture(scope="module")
def pg():
    import torch.distributed as dist
    with socket.socket() as s:
        s.bind(("127.0.0.1", 0))
        port = s.getsockname()[1]
    dist.init_process_group("nccl", init_method=f"tcp://127.0.0.1:{port}", rank=0, world_size=1)
    yield dist
    dist.destroy_process_group()


def oracle_bucket(before, r, k, levels, q_seed, select, sel_seed):
    n = before.size
    if select == "randk":
        if levels:
            idx, codes, norms, new_res, val = oracle.ef_randk_qsgd(before, r, k, sel_seed, levels=levels, group=64,
                                                                   qsgd_seed=q_seed)
        else:
            idx, val, new_res = oracle.ef_randk(before, r, k, sel_seed)
    elif levels:
        idx, codes, norms, new_res, val = oracle.ef_topk_qsgd(before, r, k, levels=levels, group=64, seed=q_seed)
    else:
        idx, val, new_res = oracle.ef_topk(before, r, k)
    out = np.zeros(n, F32)
    if levels:
        oracle.decompress_scatter(oracle.KIND_QSGD, idx, k, 0, codes, norms, None, 64, levels, F32(1.0), True, out)
    else:
        oracle.decompress_scatter(oracle.KIND_F32, idx, k, 0, val, None, None, 0, 0, F32(1.0), True, out)
    return out, new_res


@pytest.mark.parametrize("select,levels,deferred,overlap", [("topk", 127, True, True), ("topk", 0, False, True),
                                                             ("randk", 15, True, True), ("topk", 127, True, False)])
def test_ddp_hook_world_size_one(pg, select, levels, deferred, overlap):
    import torch
    from torch.nn.parallel import DistributedDataParallel as DDP
    from gradient_compression_ddp_amd.ddp_hook import CompressionHookState, ef_compress_hook

    torch.manual_seed(0)
    model = torch.nn.Sequential(torch.nn.Linear(256, 512), torch.nn.ReLU(), torch.nn.Linear(512, 512),
                                torch.nn.ReLU(), torch.nn.Linear(512, 64)).cuda()
    ddp = DDP(model, device_ids=[0], bucket_cap_mb=0.5, gradient_as_bucket_view=True)
    state = CompressionHookState(ratio=0.02, qsgd_levels=levels, select=select, deferred=deferred, seed=3,
                                 overlap=overlap)
    state.capture = []
    ddp.register_comm_hook(state, ef_compress_hook)
    gen = torch.Generator(device="cuda").manual_seed(1)
    for _ in range(3):
        x = torch.randn(32, 256, device="cuda", generator=gen)
        ddp.zero_grad(set_to_none=False)
        ddp(x).square().mean().backward()
        torch.cuda.synchronize()
    # every iteration hands at least one bucket to the hook; DDP regroups its buckets after
    # the first iteration (a regrouped bucket starts a new state), and later buckets carry
    # their residual from step to step
    assert len(state.capture) >= 3 and max(step for _, step, _, _ in state.capture) >= 1
    residuals = {}
    for index, step, before, after in state.capture:
        b = before.cpu().numpy()
        r = residuals.get((index, b.size), np.zeros(b.size, F32))
        k = state.k_for(b.size)
        sel_seed, q_seed = state.seeds(index, step)
        want, new_res = oracle_bucket(b, r, k, levels, q_seed, select, sel_seed)
        assert_bits_equal(after.cpu().numpy(), want, f"bucket {index} step {step}")
        residuals[(index, b.size)] = new_res
    # the hook's residuals, once flushed, are the oracle's
    state.flush()
    torch.cuda.synchronize()
    for index, bs in state.buckets.items():
        assert_bits_equal(bs.residual.cpu().numpy(), residuals[(index, bs.n)], f"bucket {index} residual")
