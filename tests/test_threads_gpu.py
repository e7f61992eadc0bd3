"""The library keeps no state between calls: two host threads calling
``moe_forward`` at the same time, each on its own HIP stream of the one GPU
with its own workspace and outputs, get exactly the bits that one thread gets
calling alone.  ctypes releases the interpreter lock for the length of every
foreign call, so the two threads' host code (argument checks, the per-call
device query, kernel-attribute setting and launches) runs concurrently."""
import threading

import pytest
import torch

from mixture_experts_layer_15_amd import binding as B
from mixture_experts_layer_15_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"

CASES = [
    # bf16 with many rows per expert (128 x 512 tiles), and FP8 weights on an
    # expert-parallel block: different kernel instantiations in the two threads
    synth.WORKLOADS["prefill"].replace(name="thr_bf16_T1000_d640_E32_k4_F512", T=1000, d=640,
                                       E=32, num_local=32, k=4, F=512, seed=81),
    synth.WORKLOADS["dsv3_rank"].replace(name="thr_fp8_T1500_d512_E16_local4-11_k4_F512",
                                         T=1500, d=512, E=16, num_local=8, expert_begin=4, k=4,
                                         F=512, seed=82),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load_library()


class Runner:
    """One problem's inputs, workspace and outputs; run() calls moe_forward
    `reps` times on `stream` and returns the last outputs on the host."""

    def __init__(self, wl):
        pr = synth.make_problem(wl)
        self.wl = wl
        self.p = B.problem(wl.T, wl.d, wl.E, wl.k, wl.F, wl.expert_begin, wl.num_local, wl.act,
                           wl.weight)
        self.g = {n: (None if getattr(pr, n) is None else getattr(pr, n).to(DEV))
                  for n in ("x", "w_router", "bias", "w_gate", "w_up", "w_down", "s_gate", "s_up",
                            "s_down")}
        self.ws = B.workspace(self.p, B.MOE_CALL_FORWARD, DEV)
        T, E, k, d = wl.T, wl.E, wl.k, wl.d
        self.o = dict(out=torch.empty((T, d), dtype=pr.x.dtype, device=DEV),
                      logits=torch.empty((T, E), dtype=torch.float32, device=DEV),
                      topk_idx=torch.empty((T, k), dtype=torch.int32, device=DEV),
                      slot_pos=torch.empty((T * k,), dtype=torch.int32, device=DEV))

    def run(self, stream, reps):
        g = self.g
        for _ in range(reps):
            B.moe_forward(self.p, x=g["x"], w_router=g["w_router"], router_bias=g["bias"],
                          w_gate=g["w_gate"], w_up=g["w_up"], w_down=g["w_down"],
                          s_gate=g["s_gate"], s_up=g["s_up"], s_down=g["s_down"], ws=self.ws,
                          stream=stream, **self.o)
        stream.synchronize()
        return {n: t.cpu() for n, t in self.o.items()}


def test_two_threads_on_two_streams_give_single_thread_bits():
    runners = [Runner(wl) for wl in CASES]
    torch.cuda.synchronize()  # uploads done before other streams read them
    alone = [r.run(torch.cuda.Stream(), 1) for r in runners]
    for rep in range(3):
        streams = [torch.cuda.Stream() for _ in runners]
        got = [None, None]
        errors = []
        start = threading.Barrier(len(runners))

        def work(i):
            try:
                start.wait()
                got[i] = runners[i].run(streams[i], 10)
            except Exception as e:  # reported below, in the main thread
                errors.append(e)

        threads = [threading.Thread(target=work, args=(i,)) for i in range(len(runners))]
        for t in threads:
            t.start()
        for t in threads:
            t.join(timeout=120)
        assert not any(t.is_alive() for t in threads), "a thread did not finish"
        assert not errors, errors
        for i, r in enumerate(runners):
            for n in alone[i]:
                assert torch.equal(got[i][n], alone[i][n]), (r.wl.name, n, rep)
    print("two threads: outputs equal to single-thread bits", flush=True)
