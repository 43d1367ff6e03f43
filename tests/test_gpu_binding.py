"""The Python binding's checks of caller-provided tensors: the C calls take
raw pointers and cannot see tensor sizes, so a tensor smaller than the extent
a call reads or writes is refused before anything is launched."""
import pytest
import torch

pytestmark = pytest.mark.gpu

tk = pytest.importorskip("moe_routing_amd")


def test_short_or_misplaced_tensors_are_refused():
    dev = torch.device("cuda:0")
    T, E, k, H = 64, 16, 2, 256
    logits = torch.randn((T, E), device=dev)
    opts = tk.RouteOpts(score=tk.TK_SCORE_SOFTMAX)
    with pytest.raises(ValueError):
        tk.tk_route(logits, None, k, opts, torch.empty((T, k - 1), dtype=torch.int32, device=dev))
    with pytest.raises(ValueError):
        tk.tk_route(logits, torch.zeros(E - 1, device=dev), k, opts)
    with pytest.raises(ValueError):
        tk.tk_route(logits, torch.zeros(E), k, opts)                       # bias on the host
    idx, w = tk.tk_route(logits, None, k, opts)
    with pytest.raises(ValueError):
        tk.tk_map(idx, E, pos=torch.empty(T * k - 1, dtype=torch.int32, device=dev))
    counts, offsets, pos, row_src = tk.tk_map(idx, E)
    x = torch.randn((T, H), device=dev).to(torch.bfloat16)
    with pytest.raises(ValueError):
        tk.tk_expand_quant(x, pos, tk.TK_EXPAND_FP8_E4M3_1X128, T * k,
                           scales=torch.empty((T * k, 1), dtype=torch.float32, device=dev))
    y = torch.randn((T * k, H), device=dev).to(torch.bfloat16)
    with pytest.raises(ValueError):
        tk.tk_reduce(y, pos, w, torch.empty((T - 1, H), dtype=torch.bfloat16, device=dev))
    with pytest.raises(ValueError):
        tk.tk_quant(x, tk.TK_QUANT_FP4_1X32, torch.empty((T, H // 2 - 1), dtype=torch.uint8,
                                                         device=dev))
    h = torch.randn((128, 256), device=dev).to(torch.bfloat16)
    with pytest.raises(ValueError):
        tk.tk_swiglu_quant_t(h, out_t=torch.empty((128, 127), dtype=torch.uint8, device=dev))
    torch.cuda.synchronize()
