"""The hot path under HIP graph capture: bf16 attention, an 8-chunk ring step
with its merge, the fused ring, per-tensor fp8 quantise-and-attend and
residual_diff_noalloc, captured once into a graph on a side stream and
replayed three times, with eager work and synchronisations between the
replays. Every kernel is deterministic, so every replay must equal the eager
results bit for bit. (The library calls no hipMemsetAsync and allocates
nothing; outputs and the stream's workspace exist before the capture.)"""

import pytest
import torch

import diffusion_transformer_attention_flash_amd as dta
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _same(a, b):
    if a.dtype == torch.bfloat16:
        a, b = a.view(torch.int16), b.view(torch.int16)
    return torch.equal(a, b)


def test_hot_path_replays_bitwise_under_graph_capture():
    print("CASE graph capture of the FLUX step", flush=True)
    c = workloads.CONFIGS["flux_1024"]
    c3 = workloads.CONFIGS["flux_1024_chunked"]
    c5 = workloads.CONFIGS["flux_1024_fp8"]
    B, H, N, D = c["B"], c["H"], c["N"], c["D"]
    scale = D ** -0.5
    q, k, v = workloads.workload_qkv("flux_1024", device=DEV)
    lens = workloads.chunk_lengths(c3["config"], N, c3["n_chunks"], c3["min_chunk"])
    chunks = workloads.split_kv(k, v, lens)
    ra, rb = workloads.residual_pair(c5["config"], c5["residual_shape"], c5["residual_noise"],
                                     device=DEV)
    n = len(lens)
    out = {
        "o": torch.empty_like(q), "lse": torch.empty((B, H, N), device=DEV),
        "op": torch.empty((n, B, H, N, D), dtype=torch.bfloat16, device=DEV),
        "lp": torch.empty((n, B, H, N), device=DEV),
        "om": torch.empty_like(q), "lm": torch.empty((B, H, N), device=DEV),
        "or": torch.empty_like(q), "lr": torch.empty((B, H, N), device=DEV),
        "q8": torch.empty(q.shape, dtype=torch.uint8, device=DEV),
        "k8": torch.empty(q.shape, dtype=torch.uint8, device=DEV),
        "v8": torch.empty(q.shape, dtype=torch.uint8, device=DEV),
        "ds": torch.empty(3, device=DEV),
        "o8": torch.empty_like(q), "l8": torch.empty((B, H, N), device=DEV),
        "rd": torch.empty((), device=DEV),
    }

    def step():
        dta.attn_fwd(q, k, v, scale, o=out["o"], lse=out["lse"])
        for i, (kc, vc) in enumerate(chunks):
            dta.attn_fwd(q, kc, vc, scale, o=out["op"][i], lse=out["lp"][i])
        dta.attn_merge(out["op"], out["lp"], o=out["om"], lse=out["lm"])
        dta.attn_fwd(q, chunks[0][0], chunks[0][1], scale, o=out["or"], lse=out["lr"])
        for kc, vc in chunks[1:]:
            dta.attn_fwd_accum(q, kc, vc, out["or"], out["lr"], scale)
        dta.fp8_quant_per_tensor_multi([q, k, v], [out["q8"], out["k8"], out["v8"]], out["ds"])
        dta.attn_fwd_fp8(out["q8"], out["k8"], out["v8"], out["ds"], scale,
                         o=out["o8"], lse=out["l8"])
        dta.residual_diff_noalloc(ra, rb, out["rd"])

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                                   # eager, on the capture stream
        dta.workspace(torch.device(DEV))         # that stream's workspace exists
    s.synchronize()
    eager = {name: t.clone() for name, t in out.items()}

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in out.values():                   # eager work between the replays
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t in out.items():
            assert _same(t, eager[name]), "replay %d: %s differs from eager" % (rep, name)
