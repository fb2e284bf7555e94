"""moe_expert_ffn_noalloc (the FFN with the library's static scratch array as
its workspace) against moe_expert_ffn with a caller workspace, through the C
ABI: the same kernels run on the same inputs, so the per-route outputs must be
identical bit for bit.  (With int4 weights and T > 32 the workspace call runs
the grouped GEMM on a second stream beside the streaming kernels, the no-alloc
call runs both on one stream: the comparison also shows that the overlap
changes no result.)  Calls in a row on one device, each smaller than the one
before (the array keeps the previous call's contents), then a third format; a
call too large for the array is rejected before anything runs."""
import ctypes

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

G = synth.GEMMA


def gemma_layer(lib, fmt, seed):
    """One Gemma-shaped layer's pool (128 experts packed by the library, slot
    table reversed) and its weights' slot size."""
    E, H, FF = G["E"], G["H"], G["FF"]
    dev = torch.device("cuda")
    sb = lib.expert_bytes(fmt, H, FF)
    pool = torch.empty(E * sb, dtype=torch.uint8, device=dev)
    w13, w2 = synth.layer_weights_cuda(seed, 0, E, H, FF, dev)
    slot_of = np.arange(E, dtype=np.int32)[::-1].copy()
    for e in range(E):
        s = int(slot_of[e])
        lib.pack_expert(fmt, w13[e].view(torch.int16), w2[e].view(torch.int16), pool[s * sb:(s + 1) * sb])
    del w13, w2
    return pool, sb, torch.from_numpy(slot_of).to(dev)


def both_ways(lib, pool, sb, slot_d, fmt, T, zipf, seed):
    from expert_ffn_amd.layer import MoeLayer
    E, k, H, FF = G["E"], G["k"], G["H"], G["FF"]
    print(f"[case] noalloc fmt={fmt} T={T} zipf={zipf}", flush=True)
    dev = torch.device("cuda")
    logits = torch.from_numpy(synth.logits(seed, 0, T, E, zipf)).to(dev)
    x = torch.from_numpy(synth.x_bf16(seed, 0, T, H).view(np.int16)).to(dev).view(torch.bfloat16)
    ml = MoeLayer(E, k, H, FF, fmt, T, device=dev).bind(pool, sb, slot_d)
    ml.route(logits)
    ml.out_routes.fill_(7.0)
    ml.ffn(x)
    torch.cuda.synchronize()
    kept = int(ml.offsets[E].item())
    want = ml.out_routes[:kept].clone()
    got = torch.full_like(ml.out_routes, -3.0)
    lib.expert_ffn_noalloc(pool, sb, slot_d, E, H, FF, fmt, 0, x, k, ml.offsets, ml.sorted_route[:T * k],
                           got[:T * k])
    torch.cuda.synchronize()
    assert kept > 0
    assert torch.equal(got[:kept], want), f"fmt={fmt} T={T}: no-alloc outputs differ from the workspace call's"
    assert (got[kept:] == -3.0).all(), "rows past the kept routes were written"
    print(f"    {kept} routes identical", flush=True)


def test_noalloc_matches_workspace_call():
    import expert_ffn_amd as lib
    lib.lib()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    E, k, H, FF = G["E"], G["k"], G["H"], G["FF"]
    need = lib.workspace_bytes(1024, k, E, H, FF, 2)
    assert need <= lib.NOALLOC_SCRATCH_BYTES, need
    pool, sb, slot_d = gemma_layer(lib, 2, 31)
    # 1024 tokens (grouped GEMM and streaming kernels, most of the array), then
    # 128 with Zipf routing (both families take many groups), then 16
    both_ways(lib, pool, sb, slot_d, 2, 1024, 1.1, 32)
    both_ways(lib, pool, sb, slot_d, 2, 128, 1.1, 36)
    both_ways(lib, pool, sb, slot_d, 2, 16, None, 33)
    del pool
    pool, sb, slot_d = gemma_layer(lib, 1, 34)
    both_ways(lib, pool, sb, slot_d, 1, 64, None, 35)
    # too large for the array: rejected on the host, nothing launched
    T = 4096
    assert lib.workspace_bytes(T, k, E, H, FF, 1) > lib.NOALLOC_SCRATCH_BYTES
    P = ctypes.c_void_p
    fake = P(1 << 20)
    rc = lib.lib().moe_expert_ffn_noalloc(P(pool.data_ptr()), sb, fake, E, H, FF, 1, 0, fake, 1, T, k, fake, fake,
                                          fake, 0, None)
    assert rc == 4 and "scratch" in lib.lib().moe_last_error().decode()
    torch.cuda.synchronize()
