"""The routed experts of the full-size layers element by element on samples,
through the persistent grids at their real tile counts: the DeepSeek-V3
layers (bf16 at T=8192, MXFP8 at T=16384), the pages' other layer shapes at
T=8192 in both precisions, and one GPU's EP-64 share of each (MXFP8).

Sampled routed rows (the first and last rows of the busiest expert, the rows
of the smallest non-empty expert, the last rows of an expert with 64-256
rows, and seeded random rows), four whole 32-column blocks of G, U and h, and
256 seeded columns of the expert output; each element against exact
arithmetic on the same operands (the oracle's MX rounding for MXFP8), within
the bound of the matrix cores' measured accumulation (tests/mma_rules.py),
as on the small shapes.  The rows' experts and tokens come from the oracle's
routing, which is first checked equal to the device's."""
import numpy as np
import pytest

import gen
from oracle import moe_oracle as O
from tests.mma_rules import bf16_dot, mx_dot
from tests.moe_parity import HostProblem, device_problem, to_np
from tests.test_gpu_mxfp8 import check_mx_h, mx_round

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def sample_rows(ref, R, seed, n_random=24):
    counts, off = ref["counts"], ref["offsets"]
    rng = np.random.default_rng(seed)
    hot = int(np.argmax(counts))
    rows = set(range(off[hot], off[hot] + 4)) | set(range(off[hot + 1] - 4, off[hot + 1]))
    nz = np.nonzero(counts)[0]
    small = int(nz[np.argmin(counts[nz])])
    rows |= set(range(off[small], min(off[small + 1], off[small] + 4)))
    mid = [int(e) for e in nz if 64 <= counts[e] <= 256]
    if mid:
        e = min(mid, key=lambda e: abs(int(counts[e]) - 128))
        rows |= set(range(off[e + 1] - 4, off[e + 1]))
    rows |= set(rng.choice(R, size=n_random, replace=False).tolist())
    return np.array(sorted(rows), dtype=np.int64)


# the DeepSeek-V3 layers and the pages' other layer shapes (Kimi K2.7 Code,
# GLM-5.2, Qwen3.5-397B-A17B, DeepSeek-V4-Pro; whole layers at T=8192), both precisions
N3 = ["kimi_k27", "glm52", "qwen35", "dsv4pro"]
# and one GPU's EP-64 share of each (E/64 local experts, 2,048 k rows, MXFP8)
CONFIGS = ["c3a", "c4"] + N3 + [n + "_mx" for n in N3] + ["ep64_" + n for n in ["dsv3"] + N3]


@pytest.mark.parametrize("cfg", CONFIGS)
def test_full_size_experts_elementwise(cfg):
    import mixture_experts_layer_prefix_amd as M
    D = gen.get_config(cfg)
    mx = D.prec == "mxfp8"
    say("[case] full-size element-wise", D)
    p, t, md, w = device_problem(D)
    if mx:
        w = M.prepare_mxfp8(w, md)
    hp = HostProblem(D)
    ref = hp.routing()
    _, routing = M.layer_forward(t["x"], w, md, D.prec, bias=t["bias"], keep_gu=True)
    assert np.array_equal(to_np(routing["topk_idx"]), ref["topk_idx"])
    assert np.array_equal(to_np(routing["row_token"]), ref["row_token"])
    counts, offsets, row_token, token_row, xp, xs = M.permute(routing["topk_idx"], t["x"], md, D.prec)
    h, hs = M.expert_gate_up(xp, xs, offsets, w, md, D.prec)
    o = M.expert_down(h, hs, offsets, w, md, D.prec)
    torch.cuda.synchronize()

    rows = sample_rows(ref, D.R, seed=7)
    rng = np.random.default_rng(11)
    blocks = np.sort(rng.choice(D.I // 32, size=4, replace=False))
    icols = (blocks[:, None] * 32 + np.arange(32)[None, :]).ravel()
    dcols = np.sort(rng.choice(D.d, size=256, replace=False))
    rt = torch.as_tensor(rows, device="cuda")
    gu = to_np(routing["gu"][rt]).astype(np.float64)
    Gk, Uk = gu[:, icols], gu[:, D.I + icols]
    ok = to_np(o[rt]).astype(np.float64)[:, dcols]
    if mx:
        codes = to_np(h[rt])                                        # [n][I] E4M3
        sc = to_np(hs[:, rt, :]).transpose(1, 0, 2).reshape(len(rows), D.I // 32)
    else:
        hk = to_np(h[rt]).astype(np.float64)                        # [n][I] bf16 values

    # exact operands of the sampled rows, by expert
    xr = hp.p.host_rows("x", ref["row_token"][rows])
    if mx:
        xr = mx_round(xr)
    dot = mx_dot if mx else bf16_dot
    ex = np.searchsorted(ref["offsets"], rows, side="right") - 1
    n = len(rows)
    G, dG, U, dU = (np.zeros((n, len(icols))) for _ in range(4))
    for e in np.unique(ex):
        sel = ex == e
        wg = hp.p.host_expert_rows("w_gate", int(e), icols)
        wu = hp.p.host_expert_rows("w_up", int(e), icols)
        if mx:
            wg, wu = mx_round(wg), mx_round(wu)
        G[sel], dG[sel] = dot(xr[sel], wg)
        U[sel], dU[sel] = dot(xr[sel], wu)
    half = lambda a, b: 2.0 ** -8 * np.maximum(np.abs(a), np.abs(b))
    for name, k, m, dm in (("G", Gk, G, dG), ("U", Uk, U, dU)):
        over = np.abs(k - m) - (half(k, m) + dm)
        assert np.all(over <= 0), "%s off by %.3e beyond its bound at %s" % (
            name, over.max(), np.unravel_index(np.argmax(over), over.shape))
    if mx:
        check_mx_h(G, U, dG, dU, codes[:, icols], sc[:, blocks])
        h_rows = O.e4m3_decode(codes) * np.ldexp(1.0, np.repeat(sc.astype(np.int64) - 127, 32, axis=1))
    else:
        s = O.silu(G)
        h64 = s * U
        dh = 1.1 * dG * (np.abs(U) + dU) + (np.abs(s) + 1.1 * dG) * dU + \
            2.0 ** -16 * (np.abs(s) + 1.1 * dG) * (np.abs(U) + dU)
        over = np.abs(hk[:, icols] - h64) - (half(hk[:, icols], h64) + dh)
        assert np.all(over <= 0), "h off by %.3e beyond its bound at %s" % (
            over.max(), np.unravel_index(np.argmax(over), over.shape))
        h_rows = hk
    # the down projection of the kernel's own h rows
    o_ref, do = np.zeros((n, len(dcols))), np.zeros((n, len(dcols)))
    for e in np.unique(ex):
        sel = ex == e
        wd = hp.p.host_expert_rows("w_down", int(e), dcols)
        if mx:
            wd = mx_round(wd)
        o_ref[sel], do[sel] = dot(h_rows[sel], wd)
    over = np.abs(ok - o_ref) - (half(ok, o_ref) + do)
    assert np.all(over <= 0), "o_perm off by %.3e beyond its bound at %s" % (
        over.max(), np.unravel_index(np.argmax(over), over.shape))
    say("   %d rows of %d experts (busiest %d rows), %d G/U/h columns, %d output columns: every element within its bound"
        % (n, len(np.unique(ex)), int(ref["counts"].max()), len(icols), len(dcols)))


@pytest.mark.parametrize("cfg", ["c3a", "c4"])
def test_full_size_shared_expert_elementwise(cfg):
    """The shared expert (one dense group over every token, bf16 in both
    precisions) on 24 seeded tokens: its kept G and U on four whole 32-column
    blocks within half a bf16 ulp plus the bf16 matrix cores' bound, and its
    output on 256 columns within half a bf16 ulp plus the bound carried from
    h's band (the kernel's h is not exposed: each of its values lies within
    half a bf16 ulp plus dh of the exact silu(G) U) through the down
    projection, plus the accumulation bound of that projection.  That output
    bound is coarse (about 15% of |y| at the median: the half ulps of 2,048
    h values against a cancelling sum), so it catches layout or operand
    mistakes rather than rounding ones; G and U are held tightly."""
    import mixture_experts_layer_prefix_amd as M
    D = gen.get_config(cfg)
    assert D.S == 1
    say("[case] full-size shared expert element-wise", D)
    p, t, md, w = device_problem(D)
    if D.prec == "mxfp8":
        w = M.prepare_mxfp8(w, md)
    _, routing = M.layer_forward(t["x"], w, md, D.prec, bias=t["bias"], keep_gu=True)
    y_sh = M.shared_ffn(t["x"], w, md, D.prec)
    torch.cuda.synchronize()
    rng = np.random.default_rng(13)
    toks = np.sort(rng.choice(D.T, size=24, replace=False))
    blocks = np.sort(rng.choice(D.Is // 32, size=4, replace=False))
    icols = (blocks[:, None] * 32 + np.arange(32)[None, :]).ravel()
    dcols = np.sort(rng.choice(D.d, size=256, replace=False))
    tt = torch.as_tensor(toks, device="cuda")
    gus = to_np(routing["gu_shared"][tt]).astype(np.float64)
    yk = to_np(y_sh[tt]).astype(np.float64)[:, dcols]
    hp = HostProblem(D)
    xr = hp.p.host_rows("x", toks)
    wg = hp.p.host_flat("ws_gate", 0, D.Is * D.d).reshape(D.Is, D.d)
    wu = hp.p.host_flat("ws_up", 0, D.Is * D.d).reshape(D.Is, D.d)
    wd = hp.p.host_flat("ws_down", 0, D.d * D.Is).reshape(D.d, D.Is)[dcols]
    G, dG = bf16_dot(xr, wg)
    U, dU = bf16_dot(xr, wu)
    half = lambda a, b: 2.0 ** -8 * np.maximum(np.abs(a), np.abs(b))
    for name, k, m, dm in (("G", gus[:, icols], G[:, icols], dG[:, icols]),
                           ("U", gus[:, D.Is + icols], U[:, icols], dU[:, icols])):
        over = np.abs(k - m) - (half(k, m) + dm)
        assert np.all(over <= 0), "shared %s off by %.3e beyond its bound at %s" % (
            name, over.max(), np.unravel_index(np.argmax(over), over.shape))
    s = O.silu(G)
    h64 = s * U
    dh = 1.1 * dG * (np.abs(U) + dU) + (np.abs(s) + 1.1 * dG) * dU + 2.0 ** -16 * (np.abs(s) + 1.1 * dG) * (np.abs(U) + dU)
    dh_k = 2.0 ** -8 * (np.abs(h64) + dh) + dh          # the kernel's bf16 h against h64
    y_ref = h64 @ wd.T
    carried = dh_k @ np.abs(wd).T
    _, acc = bf16_dot(np.abs(h64) + dh_k, np.abs(wd))   # accumulation bound on the kernel's operands
    over = np.abs(yk - y_ref) - (half(yk, y_ref) + carried + acc)
    assert np.all(over <= 0), "shared output off by %.3e beyond its bound at %s" % (
        over.max(), np.unravel_index(np.argmax(over), over.shape))
    say("   %d tokens, %d G/U columns, %d output columns: every element within its bound (output bound / |y| median %.2e)"
        % (len(toks), len(icols), len(dcols), float(np.median((carried + acc) / np.maximum(np.abs(y_ref), 1e-30)))))
