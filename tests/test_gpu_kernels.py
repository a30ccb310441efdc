"""Per-kernel parity of the MFMA path (needs an MI355X).

The intra-chunk step's outputs -- the fp16 operand images K~, Q' = Q~ + P' K~
and M, the bf16 hi/lo pair of P'' = P' diag(beta), and the scales of each
chunk-head record -- are decoded from the workspace and compared with the same
quantities built in fp64 from the chunked form of the gated delta rule
(oracle.chunked).  The state pass is then replayed in fp64 from the decoded
operands with its own roundings (S and R to fp16 under a per-tile power-of-two
scale) to separate the two steps: the GPU's o must match that replay far more
closely than the oracle.
"""
import numpy as np
import pytest
import torch

from hybrid_linear_attention_gdn_amd import gdn
from hybrid_linear_attention_gdn_amd.inputs import Workload, bf16_bits_to_f32, make_inputs, round_bf16_bits
from tests.helpers import oracle_for, rel_max_err, to_device

pytestmark = pytest.mark.gpu

C, D = 80, 112
# record layout (bytes): K~, Q' (5 token tiles x 3,584), P'' hi, lo (7,680 each), scales (128 fp32:
# beta[80], gamma_n), M (7 x 2,560)
KQ_BYTES, P_BYTES, CS_FLOATS = 5 * 3584, 7680, 128
REC_K, REC_Q = 0, KQ_BYTES
REC_P = 2 * KQ_BYTES
REC_PL = REC_P + P_BYTES
REC_CS = REC_PL + P_BYTES
REC_M = REC_CS + 4 * CS_FLOATS
REC_BYTES = REC_M + 7 * 2560
P_BASE = {0: 0, 1: 512, 2: 1536, 3: 3072, 4: 5120}


def _pair32(kb):
    """index of (lane, slot) in a 32-deep block in the 'pair' order: slots 0-3 are
    4g..4g+3 of the first 16, slots 4-7 the same of the second (g = lane >> 4)"""
    lane = np.arange(64)[:, None]
    j = np.arange(8)[None, :]
    g = lane >> 4
    return 32 * kb + np.where(j < 4, 4 * g + j, 16 + 4 * g + j - 4)


def _tile16(tile):
    lane = np.arange(64)[:, None]
    return 16 * tile + 4 * (lane >> 4) + np.arange(4)[None, :]


def _f16(rec, off, n):
    return rec[off:off + 2 * n].view(np.float16).astype(np.float64)


def _bf16(rec, off, n):
    return bf16_bits_to_f32(np.ascontiguousarray(rec[off:off + 2 * n]).view(np.uint16)).astype(np.float64)


def decode_kq(rec, base):
    """K~ or Q~ (80 x 112) from its fragment images"""
    X = np.zeros((C, D))
    for t in range(5):
        rows = np.broadcast_to((16 * t + (np.arange(64) & 15))[:, None], (64, 8))
        for kb in range(3):
            X[rows, _pair32(kb)] = _f16(rec, base + t * 3584 + kb * 1024, 512).reshape(64, 8)
        X[rows[:, :4], 96 + _tile16(0)] = _f16(rec, base + t * 3584 + 3072, 256).reshape(64, 4)
    return X


def decode_m(rec):
    """M (112 x 80)"""
    M = np.zeros((D, C))
    for mt in range(7):
        rows = np.broadcast_to((16 * mt + (np.arange(64) & 15))[:, None], (64, 8))
        for kb in range(2):
            M[rows, _pair32(kb)] = _f16(rec, REC_M + mt * 2560 + kb * 1024, 512).reshape(64, 8)
        M[rows[:, :4], _tile16(4)] = _f16(rec, REC_M + mt * 2560 + 2048, 256).reshape(64, 4)
    return M


def decode_p(rec, base):
    """P'' hi or lo (80 x 80), lower triangle"""
    P = np.zeros((C, C))
    for R in range(5):
        rows = np.broadcast_to((16 * R + (np.arange(64) & 15))[:, None], (64, 8))
        for kb in range((R + 1) // 2):
            P[rows, _pair32(kb)] = _bf16(rec, base + P_BASE[R] + kb * 1024, 512).reshape(64, 8)
        if R % 2 == 0:
            P[rows[:, :4], _tile16(R)] = _bf16(rec, base + P_BASE[R] + (R // 2) * 1024, 256).reshape(64, 4)
    return P


def decode(rec):
    """K~, Q', P'' (hi + lo), M, scales"""
    cs = rec[REC_CS:REC_CS + 4 * CS_FLOATS].view(np.float32).astype(np.float64)
    return (decode_kq(rec, REC_K), decode_kq(rec, REC_Q), decode_p(rec, REC_P) + decode_p(rec, REC_PL),
            decode_m(rec), cs)


def expected_chunk(inp, b, h, c):
    """fp64 K~, Q' = Q~ + P' K~, P'' = P' diag(beta), M and scales of one chunk from the chunked form."""
    from oracle.chunked import chunk_tensors
    T = inp.q.shape[1]
    sl = slice(c * C, min((c + 1) * C, T))
    n = sl.stop - sl.start
    K, Q, V = (a[b, sl, h].astype(np.float64) for a in (inp.k, inp.q, inp.v))
    rk, rq = 1 / np.linalg.norm(K, axis=1), 1 / np.linalg.norm(Q, axis=1)
    bt = 1 / (1 + np.exp(-inp.beta[b, sl, h].astype(np.float64)))
    ct = chunk_tensors(K * rk[:, None], V, Q * rq[:, None], bt, inp.g[b, sl, h].astype(np.float64))
    G, Tm = ct["G"], ct["Tm"]
    gam = np.exp(G)
    Kt, Qt = np.zeros((C, D)), np.zeros((C, D))
    Kt[:n] = -(bt * gam * rk)[:, None] * K
    Qt[:n] = (gam * rq)[:, None] * Q
    M = np.zeros((D, C))
    M[:, :n] = K.T @ np.diag(rk * np.exp(G[-1] - G)) @ Tm
    Pp = np.zeros((C, C))
    Pp[:n, :n] = ct["Pm"] @ Tm  # Pm = L o Gamma o Q^ K^T
    Qh = Qt + Pp @ Kt
    P2 = Pp.copy()
    P2[:, :n] *= bt[None, :]
    cs = np.zeros(81)
    cs[:n], cs[80] = bt, np.exp(G[-1])
    return Kt, Qh, P2, M, cs


def _run_with_ws(inp):
    q, k, v, g, beta, s0 = to_device(inp)
    B, T, H, _ = q.shape
    p = gdn.problem(B, T, H, D, D, torch.bfloat16, torch.float32)
    lay = gdn.workspace_layout(p)
    assert lay.mfma == 1 and lay.rec_bytes == REC_BYTES
    assert lay.first_range >= (T + C - 1) // C, "one chunk range: every record stays in ring slot 0"
    ws = torch.zeros(lay.total, dtype=torch.uint8, device="cuda")
    o, st = gdn.gdn_fwd(q, k, v, g, beta, s0, workspace=ws)
    torch.cuda.synchronize()
    return o.cpu().numpy(), st.cpu().numpy(), ws.cpu().numpy(), lay


def _record(ws, lay, units, u, c):
    off = lay.rec + (c * units + u) * REC_BYTES
    return ws[off:off + REC_BYTES]


def _close(got, ref, rel, label):
    """|got - ref| <= rel |ref| + 1e-5 max|ref| elementwise (rel = the operand's own rounding)."""
    err = np.abs(got - ref)
    bound = rel * np.abs(ref) + 1e-5 * np.abs(ref).max() + 1e-30
    worst = float(np.max(err / bound))
    assert worst <= 1.0, (label, worst, float(err.max()))
    return float(err.max() / max(np.abs(ref).max(), 1e-300))


def test_intra_operands_match_chunked_form():
    w = Workload("kern", 1, 3, 3, 70, "bf16", 41, state_std=0.05)
    inp = make_inputs(w)  # T = 210: chunks of 80, 80, 50 (ragged)
    o, st, ws, lay = _run_with_ws(inp)
    f16 = 2.0 ** -11  # one fp16 rounding, relative
    for h in range(3):
        for c in range(3):
            Kg, Qg, Pg, Mg, csg = decode(_record(ws, lay, 3, h, c))
            Kt, Qh, P2, M, cs = expected_chunk(inp, 0, h, c)
            eK = _close(Kg, Kt, f16, "K~")
            eQ = _close(Qg, Qh, f16, "Q'")
            eP = _close(Pg, P2, 2.0 ** -15, "P''")  # a bf16 hi/lo pair: 16 significant bits
            eM = _close(Mg, M, f16, "M")
            print(f"h={h} c={c}: max err / max  K~ {eK:.1e}  Q' {eQ:.1e}  P'' {eP:.1e}  M {eM:.1e}  "
                  f"scales {np.abs(csg[:81] - cs).max():.1e}", flush=True)
            np.testing.assert_allclose(csg[:81], cs, rtol=1e-5, atol=1e-7)


def _round_tiles(X):
    """X rounded to fp16 the way the state pass does: per block of 16 columns,
    scaled by 2^-e when its largest magnitude m leaves [2^-6, 2^15)
    (e = exponent of m - 15, m = f 2^E with f in [0.5, 1)), rounded, unscaled."""
    out = np.empty_like(X)
    for j in range(0, X.shape[1], 16):
        blk = X[:, j:j + 16]
        m = np.abs(blk).max()
        e = 0 if (m == 0 or 2.0 ** -6 <= m < 2.0 ** 15) else int(np.frexp(m)[1]) - 15
        out[:, j:j + 16] = np.ldexp(np.ldexp(blk, -e).astype(np.float16).astype(np.float64), e)
    return out


def _replay(inp, ws, lay, h, T):
    """The state pass in fp64 from the GPU's decoded operands, with the pass's own
    fp16 roundings of S and R: o and the final S^T of head h."""
    N = (T + C - 1) // C
    St = inp.state0[0, h].T.astype(np.float64)
    O = np.zeros((T, D))
    for c in range(N):
        sl = slice(c * C, min((c + 1) * C, T))
        n = sl.stop - sl.start
        Kt, Qh, P2, M, cs = decode(_record(ws, lay, inp.q.shape[2], h, c))
        V = inp.v[0, sl, h].astype(np.float64)
        S16 = _round_tiles(St)
        R16 = _round_tiles(cs[:n, None] * V + Kt[:n] @ S16)
        O[sl] = Qh[:n] @ S16 + P2[:n, :n] @ V
        St = cs[80] * St + M[:, :n] @ R16
    return O, St


@pytest.mark.parametrize("state_scale,v_scale", [(1.0, 1.0), (2.0 ** 20, 1.0), (2.0 ** -12, 2.0 ** -12)])
def test_state_pass_replayed_from_decoded_operands(state_scale, v_scale):
    """Isolates the state pass: its o equals the replay of the stated scheme to
    well within the scheme's own error against the oracle.  The replay and the
    GPU round the same operands, but from values that differ in the last fp32
    bits (fp64 here, fp32 accumulation there), so now and then one element
    rounds to the neighbouring fp16 value: sparse differences of one fp16 ulp,
    where a wrong scheme (a rounding left out, another format) differs
    everywhere.  Hence the bars: the rms difference a small fraction of the
    scheme's own rms error, the largest below the scheme's largest.  A state
    scaled by 2^20 drives S's and R's tiles above fp16's range (the rare scaled
    path); a state and values scaled by 2^-12 drive them below it."""
    w = Workload("kern2", 1, 2, 3, 70, "bf16", 43, state_std=0.05)
    inp = make_inputs(w)
    inp.state0 = (inp.state0 * state_scale).astype(np.float32)
    if v_scale != 1.0:
        inp.v = (inp.v * v_scale).astype(np.float32)
        inp.v_bits = round_bf16_bits(inp.v)
    print(f"case state x {state_scale:g}, v x {v_scale:g}", flush=True)
    o, st, ws, lay = _run_with_ws(inp)
    T = 210
    o_ref, s_ref = oracle_for(inp)
    rel_rms = lambda x, ref: float(np.sqrt(np.mean((x - ref) ** 2) / np.mean(ref ** 2)))  # noqa: E731
    for h in range(2):
        O, St = _replay(inp, ws, lay, h, T)
        ref = o_ref[0, :, h]
        e_model, r_model = rel_max_err(o[0, :, h], O), rel_rms(o[0, :, h], O)
        e_replay, r_replay = rel_max_err(O, ref), rel_rms(O, ref)
        e_gpu = rel_max_err(o[0, :, h], ref)
        print(f"h={h}: GPU vs replay max {e_model:.2e} rms {r_model:.2e}; replay vs oracle max {e_replay:.2e} "
              f"rms {r_replay:.2e}; GPU vs oracle {e_gpu:.2e}", flush=True)
        assert r_model < 0.2 * r_replay and e_model < e_replay
        assert rel_rms(st[0, h], St.T) < 0.2 * rel_rms(St.T, s_ref[0, h])
        assert e_replay < 1e-2 and e_gpu < 1e-2
        assert rel_max_err(st[0, h], s_ref[0, h]) < 1e-2
