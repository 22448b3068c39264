"""srft_attn_decode_noalloc (the attention entry point whose token-split
partials live in the library's static device scratch) against
srft_attn_decode with a caller workspace of rtq_attn_workspace_bytes(...)
bytes, through the C ABI, on consecutive calls that reuse the scratch
(needs an MI355X).  Both split a stream's tokens the same way, so their
outputs must be identical; each is also held to the oracle's bound."""
import numpy as np
import pytest

import oracle
from tests.conftest import gpu_available
from tests.parity import check_attention

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

torch = pytest.importorskip("torch")
import rotate_then_quantize_amd as rtq  # noqa: E402

DEV = "cuda"


def lm(streams, tcap):
    return (2 * streams * tcap, streams * tcap, tcap, 1)


def one_case(layers, streams, tokens, qpk, d, g, seed, rng_seed):
    rng = np.random.default_rng(rng_seed)
    strides = lm(streams, tokens)
    n = layers * 2 * streams * tokens
    rps, per = (2 * streams * tokens, layers) if layers > 1 else (0, 0)
    x = rng.standard_normal((n, d))
    x[:, rng.choice(d, 2, replace=False)] *= 15.0
    codes, scales = oracle.quant_fwd(x.astype(np.float16), g, seed, rps, per, "srft")
    q16 = rng.standard_normal((layers, streams, qpk, d)).astype(np.float16)
    ws_bytes = rtq.attn_workspace_bytes(layers, streams, tokens, qpk, d)
    print(f"case L={layers} S={streams} T={tokens} G={qpk} d={d} g={g} split workspace {ws_bytes} bytes", flush=True)
    assert ws_bytes > 0, "the case must split its streams"
    q = torch.from_numpy(q16).to(DEV)
    c = torch.from_numpy(codes).to(DEV)
    s = torch.from_numpy(scales).to(DEV)
    out_ref = torch.empty_like(q)
    out_new = torch.full_like(q, float("nan"))
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=DEV)
    lib = rtq.library()
    stream = torch.cuda.current_stream().cuda_stream
    common = (layers, streams, tokens, qpk, d, g, *strides, seed, rps, per, 1.0 / np.sqrt(d))
    st = lib.srft_attn_decode(q.data_ptr(), c.data_ptr(), s.data_ptr(), out_ref.data_ptr(), *common,
                              ws.data_ptr(), ws_bytes, stream)
    assert st == rtq.RTQ_OK, lib.rtq_status_string(st)
    st = lib.srft_attn_decode_noalloc(q.data_ptr(), c.data_ptr(), s.data_ptr(), out_new.data_ptr(), *common, stream)
    assert st == rtq.RTQ_OK, lib.rtq_status_string(st)
    torch.cuda.synchronize()
    a, b = out_ref.cpu().numpy(), out_new.cpu().numpy()
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), "no-alloc output differs from the workspace call"
    o_orc = oracle.attn_decode(q16, codes, scales, strides, layers, streams, tokens, qpk, d, g, seed, rps, per, "srft")
    worst = check_attention(b, o_orc, scales, strides, tokens, g)
    print(f"  identical to the workspace call; worst error / (2e-3 s_v) = {worst:.3f} (the bound adds 1 fp16 ulp)",
          flush=True)
    counters = (layers * streams * 4 + 255) & ~255  # the per-pair counters lead the workspace
    assert int(ws[:counters].sum()) == 0, "the workspace call leaves its counters at zero"


def test_two_calls_in_a_row_second_smaller():
    one_case(2, 3, 1500, 6, 128, 32, seed=77, rng_seed=1)   # 6 pairs, 5 splits each
    one_case(1, 2, 700, 3, 64, 32, seed=78, rng_seed=2)     # 2 pairs, 2 splits each


def test_d256_and_a_repeat():
    one_case(1, 3, 1200, 4, 256, 32, seed=79, rng_seed=3)
    one_case(1, 3, 1200, 4, 256, 32, seed=79, rng_seed=3)   # the scratch is left ready for the next call


def test_rejects_bad_arguments_before_any_launch():
    lib = rtq.library()
    q = torch.zeros((1, 1, 2, 128), dtype=torch.float16, device=DEV)
    c = torch.zeros((64, 64), dtype=torch.uint8, device=DEV)
    s = torch.zeros((64, 4), dtype=torch.float16, device=DEV)
    o = torch.empty_like(q)
    stream = torch.cuda.current_stream().cuda_stream
    args = (1, 1, 8, 2, 128, 32, 0, 32, 0, 1, 1, 0, 0, 0.1)
    assert lib.srft_attn_decode_noalloc(q.data_ptr(), c.data_ptr(), s.data_ptr(), q.data_ptr(), *args,
                                        stream) == rtq.RTQ_ERR_INVALID_ARG            # out overlaps q
    assert lib.srft_attn_decode_noalloc(q.data_ptr() + 8, c.data_ptr(), s.data_ptr(), o.data_ptr(), *args,
                                        stream) == rtq.RTQ_ERR_INVALID_ARG            # misaligned q
    bad_g = (1, 1, 8, 2, 128, 16, 0, 32, 0, 1, 1, 0, 0, 0.1)
    assert lib.srft_attn_decode_noalloc(q.data_ptr(), c.data_ptr(), s.data_ptr(), o.data_ptr(), *bad_g,
                                        stream) == rtq.RTQ_ERR_UNSUPPORTED
    torch.cuda.synchronize()
