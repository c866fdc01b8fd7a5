"""The library's calls under HIP graph capture.

A decode step or a training step is a short sequence of launches; capturing it
once in a HIP graph (torch.cuda.CUDAGraph over the current stream) and replaying
it removes the per-launch host cost.  The entry points take the caller's stream
and make no allocation, memset or synchronisation of their own, so they can be
captured when the caller supplies every output and workspace.

One graph holds a causal forward with a ragged tail, a split-KV decode and its
combine, and a causal backward.  It is replayed several times with new inputs
written between replays by ordinary eager work; after each replay every output
must equal, bit for bit, the same calls made eagerly on the same inputs.
"""
import pytest
import torch

from exact_attention_22_amd import fa

pytestmark = pytest.mark.gpu
F16 = torch.float16


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def say(msg):
    print(f"[case] {msg}", flush=True)


def same_bits(a, b):
    w = {2: torch.int16, 4: torch.int32}[a.element_size()]
    return torch.equal(a.view(w), b.view(w))


class Step:
    """Static inputs, outputs and workspaces of one forward + decode + backward."""

    def __init__(self, dev):
        B, H, N, d, Nk, S = 1, 4, 333, 128, 1500, 7
        self.shape = (B, H, N, d)
        self.S = S
        z = lambda *s, dt=F16: torch.zeros(s, dtype=dt, device=dev)
        self.q, self.k, self.v, self.g = (z(B, H, N, d) for _ in range(4))
        self.qd = z(B, H, 1, d)
        self.kd, self.vd = z(B, H, Nk, d), z(B, H, Nk, d)
        self.o, self.lse = z(B, H, N, d), z(B, H, N, dt=torch.float32)
        self.op, self.lp = z(S, B, H, 1, d, dt=torch.float32), z(S, B, H, 1, dt=torch.float32)
        self.od, self.ld = z(B, H, 1, d), z(B, H, 1, dt=torch.float32)
        self.dq, self.dk, self.dv = z(B, H, N, d), z(B, H, N, d), z(B, H, N, d)
        self.ws = z(fa.bwd_workspace_bytes(B, H, N) // 4, dt=torch.float32)

    def fill(self, seed):
        """New inputs, written in place by eager work (between replays)."""
        g = torch.Generator().manual_seed(seed)
        for t in (self.q, self.k, self.v, self.g, self.qd, self.kd, self.vd):
            t.copy_(torch.randn(t.shape, generator=g).to(F16))

    def run(self):
        fa.fwd(self.q, self.k, self.v, causal=True, out=self.o, lse=self.lse)
        fa.fwd_splitkv(self.qd, self.kd, self.vd, self.S, o_part=self.op, lse_part=self.lp)
        fa.splitkv_combine(self.op, self.lp, F16, out=self.od, lse=self.ld)
        fa.bwd(self.q, self.k, self.v, self.o, self.lse, self.g, causal=True, dq=self.dq, dk=self.dk, dv=self.dv,
               workspace=self.ws)

    def outputs(self):
        return [self.o, self.lse, self.op, self.lp, self.od, self.ld, self.dq, self.dk, self.dv]


def test_graph_replays_match_eager(dev):
    st = Step(dev)
    ref = Step(dev)
    st.fill(1)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):      # warm-up launches outside the capture
        st.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    say("capture forward + split-KV decode + combine + backward")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        st.run()
    torch.cuda.synchronize()
    for rep, seed in enumerate((11, 12, 13, 14)):
        st.fill(seed)
        ref.fill(seed)
        ref.run()                      # eager, same inputs
        torch.cuda.synchronize()
        say(f"replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        names = ["o", "lse", "o_part", "lse_part", "o_decode", "lse_decode", "dq", "dk", "dv"]
        for name, a, b in zip(names, st.outputs(), ref.outputs()):
            assert torch.isfinite(a.float()).all(), f"replay {rep}: {name} not finite"
            assert same_bits(a, b), f"replay {rep}: {name} differs from the eager call"
        print(f"[graph] replay {rep} ok", flush=True)
