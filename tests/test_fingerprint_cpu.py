"""The per-row bit fingerprint the GPU determinism test compares on every repeat
(gpu_util.checksums), checked on the CPU for the layouts it is used on: a change of
any one element's bits alters exactly its own row's sum, rows keep their order, and
the input is not copied or changed."""
import torch

from gpu_util import checksums
from linear_attention_decode_kda_amd import synth


def test_one_changed_element_changes_only_its_row():
    w = synth.WORKLOADS["tiny"]
    for dtype in (torch.float32, torch.bfloat16):
        shapes = {"o": ((w.N, w.T, w.HV, w.V), w.V), "inter_ssm": ((w.N, w.T, w.HV, w.K, w.V), w.K * w.V),
                  "conv_window": ((w.N, w.T, w.C, 3), 3 * w.C), "conv_state": ((w.N, w.C, 3), 3 * w.C)}
        for name, (shape, row) in shapes.items():
            t = torch.randn(shape).to(dtype)
            keep = t.clone()
            ref = checksums(t, row)
            assert torch.equal(t, keep), name
            assert ref.numel() == t.numel() // row, name
            g = torch.Generator().manual_seed(3)
            for _ in range(20):
                i = int(torch.randint(t.numel(), (1,), generator=g))
                u = t.clone()
                bits = u.view(-1).view(torch.int16 if dtype == torch.bfloat16 else torch.int32)
                bits[i] ^= 1 << int(torch.randint(15, (1,), generator=g))  # flip one bit
                diff = (checksums(u, row) != ref).nonzero().flatten().tolist()
                assert diff == [i // row], (name, dtype, i, diff)
