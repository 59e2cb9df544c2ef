"""spec_verify_noalloc (the library's static scratch in place of a workspace)
against spec_verify with a caller's workspace: two calls in a row on one
stream, the second with a smaller input, then both compared with what
spec_verify emits for the same inputs -- tokens and counts bit for bit, and
the lm-head's logits bit for bit. The second call runs the lm-head on the
streaming kernel with the target statistics in its epilogue, whose partials
also live in the scratch; the first call leaves larger contents behind."""

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


def to_dev(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def test_noalloc_matches_verify_two_calls(sv, dev):
    import torch
    from synth import device as sd
    # call 1: logits given, B = 16, K = 8, V = 128256 (the larger scratch)
    sigma = synth.draft_noise_sigma("stress_std3", 0.81)
    d1 = synth.sampling_inputs(71, 16, 8, 128256, 3.0, sigma)
    a1 = [to_dev(d1[k], dev) for k in ("target_logits", "draft_logits")]
    a1 += [to_dev(d1["draft_tokens"].astype(np.int32), dev), to_dev(d1["u_accept"], dev),
           to_dev(d1["u_sample"], dev)]
    # call 2: B = 1, K = 4, the lm-head 4096 -> 32000 computed first
    B2, K2, V2, dm = 1, 4, 32000, 4096
    lm = sd.normal_bf16((V2, dm), 2.0 / dm ** 0.5, 72, dev)
    hidden = sd.normal_bf16((B2 * (K2 + 1), dm), 1.0, 73, dev)
    dl2 = synth.normals(74, "noalloc.dl", (B2, K2, V2), 2.0)
    a2 = [torch.empty((B2, K2 + 1, V2), dtype=torch.float32, device=dev), to_dev(dl2, dev),
          to_dev(synth.gumbel_max_tokens(dl2, 75).astype(np.int32), dev),
          to_dev(synth.uniforms(76, "ua", (B2, K2)), dev),
          to_dev(synth.uniforms(76, "us", (B2, K2 + 1)), dev)]
    assert sv.workspace_bytes(16, 8, 128256) > sv.workspace_bytes(B2, K2, V2)

    outs = []
    for args, B, K, kw in ((a1, 16, 8, {}), (a2, B2, K2, dict(hidden=hidden, lm_head=lm))):
        out = torch.full((B, K + 1), -7, dtype=torch.int32, device=dev)
        n = torch.full((B,), -7, dtype=torch.int32, device=dev)
        sv.verify_noalloc(*args, out, n, **kw)   # no synchronization between the two calls
        outs.append((out, n))
    torch.cuda.synchronize()
    tl2_noalloc = a2[0].clone()

    for (out, n), args, kw in ((outs[0], a1, {}), (outs[1], a2, dict(hidden=hidden, lm_head=lm))):
        tl = args[0] if not kw else torch.empty_like(args[0])
        want_out, want_n = sv.verify(tl, *args[1:], **kw)
        torch.cuda.synchronize()
        assert torch.equal(out, want_out) and torch.equal(n, want_n)
        if kw:
            assert torch.equal(tl, tl2_noalloc)
        assert int(n.min()) >= 1 and int(n.max()) <= args[2].shape[1] + 1
    print(f"noalloc: call 1 mean emitted {outs[0][1].float().mean().item():.3f}, "
          f"call 2 emitted {outs[1][0].cpu().numpy().tolist()}", flush=True)
