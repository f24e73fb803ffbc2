"""The ELORA worked example (section 1.4.2 of its summary page: d = 2,
r = 1, the token 'be' with h = [1, 2], two adapters giving K = [3, 2] and
[1, 3]) through the library on the GPU, zero-padded to d = 8 (the library's
width granule).  Every value is a small integer, so each path's arithmetic is
exact and the results must equal the page's bit for bit: the fp32 path, the
bf16 path, and the bf16 prefill path (the same three tokens repeated to 258
tokens, which runs the token-tile expand on the matrix cores).  The derived
composite (2 x LoRA-1 + 1 x LoRA-2 -> [5, 3], DyMerge-LoRA section 3.1,
M1) is checked the same way."""
import json
import os

import numpy as np
import pytest
import torch

from gpu_util import make_plan
from tenant_composite_lora_amd import tclora
from tenant_composite_lora_amd import workloads as W
from test_gpu_parity import banner

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "elora_worked_example.json")
D = 8  # padded width


def _example():
    g = json.load(open(GOLDEN))
    A_t = np.zeros((2, 1, D), np.float32)
    B_t = np.zeros((2, 1, D), np.float32)
    for i, ad in enumerate(g["adapters"]):
        # the page's A (d x r) is the library's B_t^T, its B (r x d) is A_t
        A_t[i, 0, :2] = np.array(ad["B_page"], np.float32)[0]
        B_t[i, 0, :2] = np.array(ad["A_page"], np.float32)[:, 0]
    h = np.zeros(D, np.float32)
    h[:2] = g["h"]
    K_base = np.zeros(D, np.float32)
    K_base[:2] = g["K_base"]
    names = [a["name"] for a in g["adapters"]]
    dc = g["derived_composite"]
    lists = [[0], [1], [names.index(n) for n, _ in dc["pairs"]]]
    alphas = [[1.0], [1.0], [float(w) for _, w in dc["pairs"]]]
    want = [a["K"] for a in g["adapters"]] + [dc["K"]]
    return A_t, B_t, h, K_base, lists, alphas, want


@pytest.mark.parametrize("path", ["fp32", "bf16", "bf16_prefill"])
def test_elora_worked_example_bitwise(path, monkeypatch):
    monkeypatch.delenv("TCL_DISPATCH", raising=False)
    A_t, B_t, h, K_base, lists, alphas, want = _example()
    reps = 86 if path == "bf16_prefill" else 1   # 258 tokens: five token tiles
    c = W.csr_from_token_lists(lists * reps, alphas * reps, 2)
    T = c.n_tokens
    banner(f"ELORA worked example, {path}: {T} tokens")
    wd = torch.float32 if path == "fp32" else torch.bfloat16
    dev = "cuda:0"
    mod = tclora.Module(torch.from_numpy(A_t).to(dev).to(wd),
                        torch.from_numpy(B_t).to(dev).to(wd))
    x = torch.from_numpy(np.tile(h, (T, 1))).to(dev).to(wd)
    y = torch.from_numpy(np.tile(K_base, (T, 1))).to(dev)
    plan = make_plan(c)
    tclora.fused_apply(plan, [mod], [x], [y])
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    exp = np.zeros((T, D), np.float32)
    for t in range(T):
        exp[t, :2] = want[t % 3]
    print(f"  rows 0-2: {got[:3, :2].tolist()}", flush=True)
    assert np.array_equal(got.view(np.uint32), exp.view(np.uint32))
