"""lrar_backward_noalloc (the backward with no workspace argument, its query-gradient partials in
the library's per-device scratch) through the C-ABI against lrar_backward_grad, the entry point
with a caller workspace: two calls in a row, the second on a smaller input, and a key wide enough
that the scratch takes fewer workgroups."""
import numpy as np
import pytest
import torch

import parity
import transformer_depth_wise_lrar_amd as lrar
from gpu_util import f64, needs_gpu, query, say, sources
from transformer_depth_wise_lrar_amd import synth

pytestmark = [pytest.mark.gpu, needs_gpu]


def run_pair(T, d, r, n, grad, accumulate, seed):
    srcs = sources(n, T, d, "bf16", seed=seed, scale=(0.5, 4.0))
    q = query(r, seed=seed + 1)
    gdt = torch.float32 if grad == "f32" else torch.bfloat16
    dout = synth.upstream(T, d, seed + 2, device="cpu").to(gdt).cuda()
    prior = [torch.randn((T, d), generator=torch.Generator().manual_seed(seed + 3 + i))
             .to(gdt).cuda() for i in range(n)]
    ds_a = [p.clone() for p in prior] if accumulate else None
    ds_b = [p.clone() for p in prior] if accumulate else None
    say(f"[noalloc] T={T} d={d} r={r} n={n} grad={grad} accumulate={accumulate}")
    ref, dq_ref = lrar.lrar_backward_grad(srcs, q, dout, r, 1e-6, dsrc=ds_a, accumulate=accumulate)
    got, dq_got = lrar.lrar_backward_noalloc(srcs, q, dout, r, 1e-6, dsrc=ds_b,
                                             accumulate=accumulate)
    torch.cuda.synchronize()
    return ref, dq_ref, got, dq_got


def check(ref, dq_ref, got, dq_got, grad, bitwise_dq):
    for i, (a, b) in enumerate(zip(ref, got)):
        # the source gradients do not depend on the workgroup count: the same kernel, same bits
        assert torch.equal(a, b), f"dsrc[{i}] differs"
        if grad == "f32":
            parity.assert_dsrc(f64(b), f64(a), f"noalloc dsrc[{i}]")
        else:
            parity.assert_dsrc_bf16(f64(b), f64(a), f"noalloc dsrc[{i}]")
    if bitwise_dq:
        assert torch.equal(dq_ref, dq_got), "dq differs"
    ref64 = f64(dq_ref)
    bound = float(np.abs(ref64).sum())
    parity.assert_dq(f64(dq_got), ref64, bound, "noalloc dq")


@pytest.mark.parametrize("grad", ["f32", "bf16"])
def test_noalloc_matches_workspace_entry_point_twice(grad):
    """The backward workload's shape (d = 4096, r = 1024, 10 sources), then a smaller call
    (fewer rows and sources, another key width) on the same scratch: both equal the workspace
    entry point's results bit for bit (the same workgroup count)."""
    a = run_pair(4096, 4096, 1024, 10, grad, False, seed=900)
    check(*a, grad, bitwise_dq=True)
    b = run_pair(300, 1024, 64, 3, grad, True, seed=910)
    check(*b, grad, bitwise_dq=True)


def test_noalloc_wide_key_fewer_workgroups():
    """r = 4096 at 16384 rows: the workspace entry point's 2048 workgroup rows of partials
    exceed the scratch, so fewer workgroups share it; dq then sums in another fixed order and is
    held to the dq bar, the source gradients stay bit for bit."""
    a = run_pair(16384, 4096, 4096, 4, "f32", False, seed=920)
    check(*a, "f32", bitwise_dq=False)
    b = run_pair(64, 4096, 4096, 2, "f32", False, seed=930)
    check(*b, "f32", bitwise_dq=True)


@pytest.mark.parametrize("grad", ["f32", "bf16"])
def test_noalloc_element_path_twice(grad):
    """Rows the element path serves (an unaligned width, and a width past a register tile with
    an odd row stride): the one-wave-per-row backward with the scratch, twice in a row, equal to
    the workspace entry point bit for bit."""
    a = run_pair(257, 513, 200, 3, grad, False, seed=960)
    check(*a, grad, bitwise_dq=True)
    b = run_pair(70, 2561, 640, 2, grad, True, seed=970)
    check(*b, grad, bitwise_dq=True)


def test_noalloc_rejects_a_key_beyond_the_scratch():
    srcs = sources(1, 2048, 16384, "bf16", seed=940)
    q = query(16384, seed=941)
    dout = torch.zeros((2048, 16384), dtype=torch.float32, device="cuda")
    with pytest.raises(lrar.LrarError) as e:
        lrar.lrar_backward_noalloc(srcs, q, dout, 16384, 1e-6)
    assert e.value.status == lrar.LRAR_ERR_UNSUPPORTED
