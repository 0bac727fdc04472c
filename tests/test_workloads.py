"""The seeded input generator: shapes, dtypes, determinism, key lengths."""
import math

import torch

from online_softmax_03_amd import workloads as W


def test_five_workloads_as_specified():
    names = [w.name for w in W.WORKLOADS]
    assert len(names) == 5 and len(set(names)) == 5
    t, c2, c3, c4, c5 = W.WORKLOADS
    assert (t.B, t.H, t.N, t.d, t.in_dtype, t.causal, t.block_c) == (1, 1, 256, 64, "f32", False, 64)
    assert (c2.B, c2.H, c2.N, c2.d, c2.in_dtype, c2.out_dtype, c2.causal) == (4, 16, 2048, 64, "bf16", "f32", False)
    assert (c3.B, c3.H, c3.N, c3.d, c3.in_dtype, c3.causal) == (2, 32, 8192, 128, "bf16", True)
    assert (c4.B, c4.H, c4.N, c4.d, c4.causal, c4.q_dist) == (1, 8, 32768, 128, True, ("normal", 2.0))
    assert (c5.B, c5.H, c5.N, c5.d, c5.in_dtype, c5.key_padding) == (8, 16, 4096, 64, "f16", True)
    assert c5.q_dist == ("normal", 3.0) and c5.v_dist == ("uniform", -1.0, 1.0)
    assert c3.scale == float(torch.tensor(1 / math.sqrt(128), dtype=torch.float32))
    assert c3.nominal_flops() == 4 * 2 * 32 * 8192 ** 2 * 128 / 2


def test_generation_is_deterministic_and_typed():
    w = W.WORKLOADS[4].with_shape(B=4, H=2, N=64)
    a, b = W.generate(w), W.generate(w)
    for n in ("q", "k", "v", "mask", "lens"):
        assert torch.equal(a[n], b[n])
    assert a["q"].dtype == torch.float16 and a["q"].shape == (4, 2, 64, 64) and a["q"].is_contiguous()
    assert a["mask"].dtype == torch.uint8 and a["mask"].shape == (4, 64)
    assert a["lens"][0] == 0 and a["lens"][-1] == 64
    assert torch.equal(a["mask"].sum(1), a["lens"].to(torch.uint8).to(torch.int64))
    v = a["v"].float()
    assert v.min() >= -1 and v.max() <= 1
    c = W.generate(w, seed=99)
    assert not torch.equal(a["q"], c["q"])


def test_values_are_exact_in_the_input_dtype():
    w = W.WORKLOADS[2].with_shape(B=1, H=1, N=32)
    x = W.generate(w)
    assert x["q"].dtype == torch.bfloat16
    assert torch.equal(x["q"].float().to(torch.bfloat16), x["q"])


def test_every_hip_source_belongs_to_a_profiled_kernel():
    """Each file under csrc/ is part of some kernel's source hash, so a change
    to it invalidates that kernel's committed traffic figures (apart from the
    host-only error texts)."""
    import glob
    import os

    from online_softmax_03_amd import profiling
    listed = {f for files in profiling.KERNEL_SOURCES.values() for f in files} | set(profiling.HOST_ONLY_SOURCES)
    present = {os.path.basename(f) for f in glob.glob(os.path.join(profiling.PKG, "csrc", "*"))}
    assert present == listed
