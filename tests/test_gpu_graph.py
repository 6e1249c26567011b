"""A whole sampling call captured in a HIP graph (GPU only).

cfm_sample synchronises nothing with the host and allocates nothing, so a caller
can capture it (VoiceHub "Diffusion and flow TTS optimization", section "Static
shapes and CUDA graphs"; vox-serve "Adding a Model", graph-capture rules). The
graph holds a device-to-device copy and kernels only. Each replay, with eager
work of the same sampler between replays, must give the eager call's bits.
"""
import numpy as np
import pytest

import synth
from tests.helpers import config_for, dev

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import flow_matching_tts_amd as F
    F.load()


@pytest.mark.parametrize("name,kw,opts", [
    ("locdit_tail", dict(n_requests=16, n_steps=4, n_layers=2), {}),
    ("mel_dit", dict(n_layers=2, n_frames=200, n_requests=2, n_steps=3), {}),
    ("varlen_masked", dict(n_layers=2, n_frames=300, n_requests=3, n_steps=3, varlen=(60, 300)),
     dict(guidance_mode="adaptive", adaptive=(0.5, 1, 1))),
    ("mel_dit", dict(n_layers=4, n_frames=200, n_requests=2, n_steps=6), dict(cache={})),
])
def test_graph_replays_equal_the_eager_call(name, kw, opts):
    import flow_matching_tts_amd as F
    s = synth.workload(name).replace(**kw)
    W, I = synth.make_weights(s, 701), synth.make_inputs(s, 702)
    smp = F.Sampler(config_for(s), W)
    x0, cond = dev(I["x0"]), dev(I["cond"])
    mask, spk = dev(I["mask"]), dev(I["spk"])
    out = torch.empty_like(x0)
    call = lambda o: smp.sample(x0, cond, mask=mask, spk=spk, n_steps=s.n_steps, guidance=s.guidance, out=o,
                                **opts)
    call(out)
    torch.cuda.synchronize()
    eager = out.clone()
    graph = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            call(out)
    torch.cuda.current_stream().wait_stream(stream)
    other = torch.empty_like(x0)
    for i in range(3):
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), i
        call(other)                     # eager work of the same context between replays
        torch.cuda.synchronize()
        assert torch.equal(other, eager), i
