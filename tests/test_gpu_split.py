"""GPU parity of attn_fwd_split (attn_fwd with a partial last round of query
tiles cut along K/V across the idle compute units) against the float64
oracle, through the C ABI; and its agreement with attn_fwd.

The cut depends on the device's compute-unit count; `_plan` restates the
schedule include/dta.h documents, so that each case states whether, and how
finely, it cuts.
"""

import math

import pytest
import torch

import diffusion_transformer_attention_flash_amd as dta
import oracle
import workloads
from helpers import assert_bf16_attention

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _plan(B, H, Nq, Nkv):
    """(items run whole, cut items, ranges, shortest range in tiles), or None
    when the call is plain attn_fwd."""
    C = min(torch.cuda.get_device_properties(0).multi_processor_count, 256)
    n = B * H * math.ceil(Nq / 256)
    n_tiles = math.ceil(Nkv / 64)
    r = n % C
    if r == 0:
        return None
    n_wg = min(C, 2 * r)
    lmin = r * n_tiles // n_wg
    if lmin < 16 or (n_tiles - 1 + lmin - 1) // lmin + 1 > 3:
        return None
    return n - r, r, n_wg, lmin


def _case(name, **kw):
    print("CASE", name, kw, flush=True)


SHAPES = [
    (1, 1, 256, 2048),       # one query tile in two pieces
    (1, 3, 500, 2600),       # ragged Nq and Nkv (41 tiles, the last of 40 keys)
    (2, 4, 2304, 2100),      # 72 query tiles, two pieces each, ragged tail
    (1, 8, 4608, 2048),      # 144 query tiles over all ranges: up to three pieces
    (1, 24, 4608, 4608),     # FLUX.1-dev 1024^2: 256 whole, 176 cut
]


@pytest.mark.parametrize("B,H,Nq,Nkv", SHAPES)
def test_split_shapes_all_rows(B, H, Nq, Nkv):
    plan = _plan(B, H, Nq, Nkv)
    _case("split", B=B, H=H, Nq=Nq, Nkv=Nkv, plan=plan)
    q, k, v = workloads.make_qkv(51, B, H, Nq, Nkv, 128, device=DEV)
    scale = 128 ** -0.5
    o, lse = dta.attn_fwd_split(q, k, v, scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(q.cpu(), k.cpu(), v.cpu(), scale)
    assert_bf16_attention(o, lse, o_ref, lse_ref, "split %s" % ((B, H, Nq, Nkv),))


def test_split_flux_workload_all_rows():
    # The FLUX.1-dev 1024^2 workload itself (QK-normed), every row.
    c = workloads.CONFIGS["flux_1024"]
    _case("split flux_1024", **{k: c[k] for k in ("B", "H", "N", "D")})
    q, k, v = workloads.workload_qkv("flux_1024", device=DEV)
    scale = c["D"] ** -0.5
    o, lse = dta.attn_fwd_split(q, k, v, scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(q.cpu(), k.cpu(), v.cpu(), scale)
    assert_bf16_attention(o, lse, o_ref, lse_ref, "split flux_1024 (all rows)")


@pytest.mark.parametrize("B,H,Nq,Nkv", SHAPES)
def test_split_agrees_with_attn_fwd(B, H, Nq, Nkv):
    """Whole query tiles run attn_fwd's arithmetic: bit-identical. A cut tile
    rounds P to bf16 against each piece's own reference max and regroups
    float32 sums. Each side's O then errs by at most 2^-8 sum_j p_j |v_j| / l
    (P rounding, half a bf16 ulp per weight) plus 2^-8 |O| (the final
    rounding), so the two differ by at most 2^-7 (A + |O|), where A is
    attention over |V|. LSE is summed from unrounded weights in float32."""
    plan = _plan(B, H, Nq, Nkv)
    _case("split vs attn_fwd", B=B, H=H, Nq=Nq, Nkv=Nkv, plan=plan)
    q, k, v = workloads.make_qkv(53, B, H, Nq, Nkv, 128, device=DEV, q_gain=2.0)
    scale = 128 ** -0.5
    o1, l1 = dta.attn_fwd(q, k, v, scale)
    o2, l2 = dta.attn_fwd_split(q, k, v, scale)
    torch.cuda.synchronize()
    n_qt = math.ceil(Nq / 256)
    n_whole = plan[0] if plan else B * H * n_qt
    # query tile t = (b*H + h) * n_qt + qt; rows of whole tiles first
    rows = torch.zeros(B * H, n_qt * 256, dtype=torch.bool, device=DEV)
    for t in range(n_whole):
        rows[t // n_qt, (t % n_qt) * 256:(t % n_qt + 1) * 256] = True
    whole = rows[:, :Nq].reshape(B, H, Nq)
    a, b = o1.float(), o2.float()
    assert torch.equal(o1[whole].view(torch.int16), o2[whole].view(torch.int16))
    assert torch.equal(l1[whole], l2[whole])
    cut = ~whole
    if plan is None:
        assert not cut.any()
        return
    assert cut.any()
    o_abs, _ = dta.attn_fwd(q, k, v.abs(), scale)
    bound = 2.0 ** -7 * (o_abs.float()[cut] + a[cut].abs()) + 1e-6
    err = (a[cut] - b[cut]).abs()
    assert (err <= bound).all(), (err / bound).max().item()
    lerr = (l1[cut] - l2[cut]).abs()
    assert (lerr <= 1e-5 * l1[cut].abs().clamp(min=1.0)).all(), lerr.max().item()
    print("cut rows: O max diff %.3e, LSE max diff %.3e" % (err.max().item(), lerr.max().item()))


def test_split_repeats_bitwise_and_resets_its_counters():
    """The pieces' counters return to zero: the same call gives the same bits
    before and after calls of other shapes on the same workspace, and the
    counter region is zero afterwards."""
    _case("split repeats")
    shapes = [(1, 24, 4608, 4608), (1, 3, 500, 2600), (1, 8, 4608, 2048)]
    data = [workloads.make_qkv(55 + i, *s, 128, device=DEV) for i, s in enumerate(shapes)]
    first = [dta.attn_fwd_split(*d, 128 ** -0.5) for d in data]
    for rep in range(5):
        for d, (o0, l0) in zip(data, first):
            o, l = dta.attn_fwd_split(*d, 128 ** -0.5)
            torch.cuda.synchronize()
            assert torch.equal(o.view(torch.int16), o0.view(torch.int16)), rep
            assert torch.equal(l, l0), rep
    ws = dta.split_workspace(torch.device(DEV))
    assert int(ws[:4096].count_nonzero()) == 0
