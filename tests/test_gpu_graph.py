"""lq_gemv captured in a HIP graph: every path (one launch; slice-major
kernel and reduction; preparation, product and reduction for 6 - 16 tokens)
replayed several times, with eager calls of other token counts on the same
workspace between the replays, each replay equal bit for bit to the eager
call (the kernels are deterministic and clear nothing with memset, so a
replay must not depend on what earlier calls left in the workspace)."""
import numpy as np
import pytest

from bit_lifted_gemv_amd import synth

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    from bit_lifted_gemv_amd import lq
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lq.load_library()
    return torch.device("cuda:0")


GRAPH_CASES = [  # (m, K, B): the path each one takes
    (8192, 19456, 1),    # one launch (19 slices)
    (2048, 68096, 1),    # slice-major kernel and its reduction (67 slices)
    (4096, 28672, 1),    # one launch with 16 waves (28 slices)
    (8192, 19456, 4),    # slice-major kernel and its reduction, four tokens
    (8192, 19456, 16),   # preparation, product with register-held operands, reduction
    (4104, 9216, 7),     # the same at 7 tokens, a ragged last row tile
]


@pytest.mark.parametrize("m,K,B", GRAPH_CASES)
def test_gemv_graph_replays_match_eager(dev, m, K, B):
    from bit_lifted_gemv_amd import lq
    rng = np.random.default_rng(m + K + B)
    ldw = ((K + 31) // 32 + 3) // 4 * 4
    w = torch.from_numpy(synth.random_sign_words(rng, m, K, ldw=ldw).view(np.int32)).to(dev)
    s = torch.from_numpy(rng.uniform(0.01, 0.03, m).astype(np.float32)).to(dev)
    a = torch.from_numpy(rng.standard_normal((B, K)).astype(np.float32)).to(dev)
    other = [torch.from_numpy(rng.standard_normal((b, K)).astype(np.float32)).to(dev)
             for b in (1, 5, 16)]
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    out = torch.empty(B, m, device=dev)
    with torch.cuda.stream(st):
        ref = lq.gemv(w, s, a, K).clone()
        lq.gemv(w, s, a, K, out=out)            # the workspace exists before capture
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=st):
            lq.gemv(w, s, a, K, out=out)
        for r in range(3):
            out.zero_()
            gr.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref), f"replay {r}"
            for ao in other:                    # eager calls over the same workspace
                lq.gemv(w, s, ao, K)
            torch.cuda.synchronize()


@pytest.mark.parametrize("m,n,d,D,B", [(8192, 8192, 8, 19, 16), (1000, 4096, 8, 16, 7)])
def test_parts_path_graph_replays_match_eager(dev, m, n, d, D, B):
    """lq_lift_parts + lq_gemv_parts captured together: three replays, eager
    calls with other token counts on the same workspace in between, each
    replay equal bit for bit to the eager pair."""
    from bit_lifted_gemv_amd import lq
    L = synth.make_layer(m, n, d, D, B, seed=m + B, dtype="bf16")
    dl = lq.DeviceLayer.from_synth(L, device=dev)
    a = lq.to_torch_16(L.a, "bf16").to(dev)
    others = [lq.to_torch_16(synth.make_layer(64, n, d, D, b, seed=b, dtype="bf16").a,
                             "bf16").to(dev) for b in (6, 16)]
    img = torch.empty(lq.lift_parts_size(L.K), dtype=torch.uint8, device=dev)
    out = torch.empty(B, m, device=dev)
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        ref = dl.forward(a, path="parts").clone()
        lq.lift_parts(a, dl.t_inv, dl.M, d, D, out=img)
        lq.gemv_parts(dl.w, dl.s, img, L.K, B, out=out)   # the workspace exists before capture
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=st):
            lq.lift_parts(a, dl.t_inv, dl.M, d, D, out=img)
            lq.gemv_parts(dl.w, dl.s, img, L.K, B, out=out)
        for r in range(3):
            out.zero_()
            img.zero_()
            gr.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref), f"replay {r}"
            for ao in others:                   # eager calls over the same workspace
                dl.forward(ao, path="parts")
            torch.cuda.synchronize()
