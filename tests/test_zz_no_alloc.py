"""qmv_chain_noalloc (barrier words held by the library, no workspace)
against qmv_chain with a caller workspace, called through the C ABI: the
same outputs bitwise (the same kernels) and within the accuracy bound of the
oracle, on two calls in a row, the second with a smaller stage list.  The
stages are decode-shaped and dependent (stage barriers inside the
persistent kernels use the barrier words), and the first list holds more
stages than one launch, so it also crosses a launch boundary; both
persistent kernels of qmv_chain are reached."""
import ctypes

import numpy as np
import pytest

import oracle
import workloads as wl

pytestmark = pytest.mark.gpu


def _decode_stages(torch, qmv, fmt, layers, tag, F):
    """q reads the layer input, k too (no wait), o reads q, gate and up read
    o (up does not wait), down reads up and is the next layer's input."""
    H = 2048
    mats = {"q": (H, H), "k": (512, H), "o": (H, H), "gate": (F, H), "up": (F, H), "down": (H, F)}
    Wd = {m: torch.from_numpy(wl.quant_weights(fmt, f"t/noalloc/{tag}/{m}", N, K)).to("cuda:0")
          for m, (N, K) in mats.items()}
    h = torch.from_numpy(wl.activations(f"t/noalloc/{tag}/h", 1, H)).to("cuda:0")[0]
    stages, outs = [], []
    for _ in range(layers):
        y = {m: torch.full((N,), float("nan"), device="cuda:0") for m, (N, _) in mats.items()}
        stages += [(Wd["q"], H, H, h, y["q"], 1), (Wd["k"], 512, H, h, y["k"], 0),
                   (Wd["o"], H, H, y["q"], y["o"], 1), (Wd["gate"], F, H, y["o"], y["gate"], 1),
                   (Wd["up"], F, H, y["o"], y["up"], 0), (Wd["down"], H, F, y["up"], y["down"], 1)]
        outs += [y[m] for m in ("q", "k", "o", "gate", "up", "down")]
        h = y["down"]
    return stages, outs


# F = 5632: the per-stage chain kernel (two-level atomic barrier words);
# F = 6144: whole 2048-column windows, the streaming kernel (flag words)
@pytest.mark.parametrize("F", [5632, 6144])
@pytest.mark.parametrize("fmt", ["q8_0", "q4_0"])
def test_chain_noalloc_equals_chain(fmt, F):
    import torch
    import bandwidth_bound_block_amd as qmv
    lib = qmv.lib()
    ws = torch.zeros(qmv.CHAIN_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    for call, layers in enumerate((12, 2)):          # 72 stages (two launches), then 12
        print(f"noalloc {fmt} F={F} call {call}: {layers} layers", flush=True)
        stages, outs = _decode_stages(torch, qmv, fmt, layers, f"{fmt}/{F}/{call}", F)
        arr = qmv.chain_stages(stages, fmt)
        rc = lib.qmv_chain(qmv.FORMATS[fmt], ctypes.cast(arr, ctypes.c_void_p), len(arr), ws.data_ptr(), ws.numel(),
                           ctypes.c_void_p(stream))
        assert rc == 0, qmv.last_error()
        torch.cuda.synchronize()
        assert int(ws.view(torch.int32)[2].item()) == 0
        ref = [y.clone() for y in outs]
        for y in outs:
            y.fill_(float("nan"))
        rc = lib.qmv_chain_noalloc(qmv.FORMATS[fmt], ctypes.cast(arr, ctypes.c_void_p), len(arr),
                                   ctypes.c_void_p(stream))
        assert rc == 0, qmv.last_error()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(ref, outs)):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), (fmt, call, i)
        # the last layer's stages against the oracle, each on its own input
        for W, N, K, x, y, _ in stages[-6:]:
            yr, S = oracle.matvec(fmt, W.cpu().numpy(), N, K, x.cpu().numpy()[None])
            err = np.abs(y.cpu().numpy().astype(np.float64) - yr[0])
            assert np.all(err <= 1e-4 * S[0] + 1e-6), (fmt, call, N, K)
