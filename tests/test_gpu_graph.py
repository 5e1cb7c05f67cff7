"""HIP graph capture of a whole decode step (mla_absorb_q, mla_decode, mla_absorb_out)
through the C ABI: the library never synchronises, allocates or writes memory with a
memset, so the step can be captured on a stream and replayed.  Every replay, with eager
work in between that overwrites the outputs, must reproduce the eager step bit for bit
(the kernels are deterministic)."""
import numpy as np
import pytest
import torch

from mla_latent_kv_lat_amd import capi, configs, synth
from mla_latent_kv_lat_amd.runner import DeviceWorkload, to_host_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    capi.library()
    return "cuda"


@pytest.mark.parametrize("case", ["balanced", "split256", "paged"])
def test_graph_replay_matches_eager_step(case):
    kw = dict(batch=6, seq_len=1500, cfg_id=60)
    if case == "paged":
        cfg = configs.PAGED_VARLEN.with_(batch=5, seq_len=2000, cfg_id=61)
    else:
        cfg = configs.V2_DECODE.with_(**kw)
    print("[case] graph replay", case, cfg.batch, cfg.seq_len, flush=True)
    lengths = np.random.default_rng(3).integers(1, cfg.seq_len + 1, size=cfg.batch).astype(np.int32)
    inp = synth.make_inputs(cfg, 0, lengths=lengths)
    w = DeviceWorkload(inp, split_tokens=256 if case == "split256" else 0, replicas=1)
    c = w.caches[0]

    def step():
        w.absorb_q(c)
        w.decode(c)
        w.absorb_out(c)

    step()
    torch.cuda.synchronize()
    ref = [to_host_f64(t) for t in (w.q_lat, w.o_lat, w.lse, w.out)]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (w.q_lat, w.o_lat, w.out):
            t.fill_(7.0)  # eager work between replays that the replay must overwrite
        w.lse.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [to_host_f64(t) for t in (w.q_lat, w.o_lat, w.lse, w.out)]
        for name, a, b in zip(("q_lat", "o_lat", "lse", "out"), got, ref):
            assert np.array_equal(a, b, equal_nan=True), (case, rep, name)
