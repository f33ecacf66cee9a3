"""jepa_encode_noalloc (the encode for callers that cannot allocate device
memory) through the C ABI against jepa_encode, whose launch sequence it runs
over a static device array instead of the context's workspace."""
import numpy as np
import pytest

from tests import helpers as H
from vision_transformer_amd import synth

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from vision_transformer_amd import _lib
    return _lib


# workloads: bf16 block-causal with CLS, q8_0 (weights dequantised in the
# tile load), and the full-size f32 ViT-Ti/14 image model (its residual GEMMs
# and attention split over workgroups with partial sums in the scratch)
CASES = [("small_blockcausal_bf16", 3, 1), ("small_tubelet2_q8_0", 2, 1), ("vit_ti14_image_f32", 3, 1)]


@pytest.mark.parametrize("name,b1,b2", CASES)
def test_noalloc_matches_encode_on_two_calls(lib, name, b1, b2):
    """Two calls in a row, the second with a smaller batch: each token map
    equals jepa_encode's (the batch as one part, as the no-allocation call
    runs it) bit for bit, and meets the oracle-parity bar against it."""
    wl, dims, _, stored = H.workload_inputs(name)
    frames = synth.make_frames(dims, b1, 93)
    ctx = lib.jepa_create(dims, stored)
    lib.jepa_set_batch_parts(ctx, 1)
    N, D = synth.n_tokens(dims), dims["dim"]
    try:
        for B in (b1, b2):
            H.say(f"encode_noalloc {name} batch {B}")
            fr = torch.from_numpy(np.ascontiguousarray(frames[:B])).cuda()
            want = torch.empty((B, N, D), device="cuda")
            got = torch.full((B, N, D), float("nan"), device="cuda")
            lib.jepa_encode(ctx, fr, B, want)
            torch.cuda.synchronize()
            lib.jepa_encode_noalloc(ctx, fr, B, got)
            torch.cuda.synchronize()
            H.check_rows(dims["act_dtype"], got.cpu().numpy(), want.cpu().numpy().astype(np.float64),
                         "noalloc vs encode")
            assert torch.equal(got, want)
            # the previous token map is forgotten
            with pytest.raises(lib.JepaError, match="JEPA_E_STATE"):
                lib.jepa_pool(ctx, "mean", torch.empty((B, D), device="cuda"))
    finally:
        lib.jepa_free(ctx)


def test_noalloc_graph_replay_and_refusals(lib):
    """Captured into a HIP graph and replayed three times with eager work in
    between, it reproduces the eager result; a batch too large for the
    static array, host frames and a missing output are refused before any
    work is enqueued."""
    wl, dims, frames, stored = H.workload_inputs("small_blockcausal_bf16")
    ctx = lib.jepa_create(dims, stored)
    try:
        B, N, D = frames.shape[0], synth.n_tokens(dims), dims["dim"]
        fr = torch.from_numpy(frames).cuda()
        tokens = torch.empty((B, N, D), device="cuda")
        lib.jepa_encode_noalloc(ctx, fr, B, tokens)
        torch.cuda.synchronize()
        want = tokens.clone()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            lib.jepa_encode_noalloc(ctx, fr, B, tokens)
        for r in range(3):
            H.say(f"encode_noalloc graph replay {r}")
            tokens.zero_()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(tokens, want)
            lib.jepa_encode(ctx, fr, B, torch.empty_like(tokens))   # eager work between replays
            torch.cuda.synchronize()
        del graph
        big = 1 + lib.NOALLOC_SCRATCH_BYTES // (N * D * 4)          # the f32 residual stream alone overflows
        with pytest.raises(lib.JepaError, match="JEPA_E_OOM"):
            lib._check(lib._lib.jepa_encode_noalloc(ctx, fr.data_ptr(), big, tokens.data_ptr(), None))
        with pytest.raises(lib.JepaError, match="JEPA_E_INVALID_ARG"):
            lib._check(lib._lib.jepa_encode_noalloc(ctx, fr.data_ptr(), B, None, None))
        with pytest.raises(ValueError):
            lib.jepa_encode_noalloc(ctx, frames, B, tokens)
    finally:
        lib.jepa_free(ctx)
