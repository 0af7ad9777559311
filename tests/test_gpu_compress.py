"""GPU parity of sl_compress against the CPU oracle.

Indices, codes and scales (the whole 112-byte record plus the fp32 scale) must
be bit-exact; the error-feedback buffer is compared bitwise as well (the design
target is 0 ulp, inside the 1e-6 relative bound, because any drift would change
later rounds' selections).
"""
import numpy as np
import pytest
import torch

import special_chunks as sc
from communication_efficient_distributed_amd import datagen
from gpu_util import assert_bitwise, note, oracle_threads, require_gpu

pytestmark = pytest.mark.gpu


def gpu_round(sl, delta_np, ef_np, beta):
    dev = torch.device("cuda:0")
    d = torch.from_numpy(np.ascontiguousarray(delta_np)).to(dev)
    e = torch.from_numpy(np.ascontiguousarray(ef_np)).to(dev)
    payload, scales = sl.compress(d, e, beta)
    torch.cuda.synchronize()
    return payload.cpu().numpy(), scales.cpu().numpy(), e.cpu().numpy()


def check_round(sl, orc, delta, ef, beta, what):
    note(f"{what}: sl_compress n={delta.size} beta={beta}")
    gp, gs, ge = gpu_round(sl, delta, ef, beta)
    op, os_, oe = orc.compress(delta, ef, beta=beta, nthreads=oracle_threads())
    assert_bitwise(gp, op, f"{what} payload")
    assert_bitwise(gs, os_, f"{what} scales")
    assert_bitwise(ge, oe, f"{what} ef")
    return oe


def test_special_chunks(orc):
    sl = require_gpu()
    gold = sc.load_golden()
    ds, es = [], []
    for case in ("E1", "E2", "E3", "E4"):
        d, e = sc.inputs(case)
        check_round(sl, orc, d, e, 0.95, f"special {case}")
        ds.append(d)
        es.append(e)
    # the four side by side in one call, plus the hand-derived bytes
    d = np.concatenate(ds)
    e = np.concatenate(es)
    note("special E1..E4 batched")
    gp, gs, ge = gpu_round(sl, d, e, 0.95)
    for c, case in enumerate(("E1", "E2", "E3", "E4")):
        for field, want in gold[case].items():
            if field == "scale":
                assert int(gs.view(np.uint32)[c]) == want
            else:
                a, b = sc.byte_range(field)
                assert gp[c, a:b].tobytes() == want, (case, field)
        assert_bitwise(ge[c * 4096:(c + 1) * 4096], sc.expected_new_ef(case), f"{case} ef")


def test_small_1m_three_rounds(orc):
    """1,048,576 params (256 chunks): lognormal groups, outliers, ef = 0,
    beta = 0.95, three rounds with fresh delta."""
    sl = require_gpu()
    n = datagen.WORKLOAD_PARAMS[datagen.SMALL_1M]
    ef = np.zeros(n, np.float32)
    factors = datagen.group_factors(n, datagen.SMALL_1M, 0)
    for rnd in range(3):
        delta = datagen.lognormal(n, datagen.SMALL_1M, 0, rnd, factors=factors).numpy()
        ef = check_round(sl, orc, delta, ef, 0.95, f"small_1m round {rnd}")


def _tricky_chunks(rng):
    """Chunks that exercise every branch of the selection."""
    chunks = []
    z = np.zeros(4096, np.float32)
    chunks.append(z.copy())                                         # all +0
    chunks.append(-z)                                               # all -0
    c = z.copy(); c[rng.choice(4096, 10, replace=False)] = 1.0; chunks.append(c)      # < 64 nonzeros
    c = z.copy(); c[rng.choice(4096, 64, replace=False)] = -2.0; chunks.append(c)     # exactly 64
    c = z.copy(); c[rng.choice(4096, 65, replace=False)] = 3.0; chunks.append(c)      # 65 equal
    chunks.append(np.full(4096, 1.25, np.float32))                  # 4096 equal
    chunks.append(np.full(4096, -7.0, np.float32))
    chunks.append(rng.integers(-3, 4, 4096).astype(np.float32))     # heavy ties
    chunks.append(rng.integers(-40, 41, 4096).astype(np.float32) * np.float32(0.5))
    den = (rng.integers(0, 1 << 23, 4096).astype(np.uint32)).view(np.float32).copy()
    chunks.append(den)                                              # denormals
    c = den.copy(); c[::7] = -0.0; chunks.append(c)
    # one binade: uniform in [1, 2) -> many entries share the level-0 bin
    chunks.append((1.0 + rng.random(4096)).astype(np.float32))
    # near-equal magnitudes differing in the last mantissa bits
    base = np.float32(3.0)
    c = np.array([np.nextafter(base, np.float32(9), dtype=np.float32)] * 4096, np.float32)
    c.view(np.uint32)[:] += rng.integers(0, 300, 4096).astype(np.uint32)
    chunks.append(c)
    # mixed: 50 loud, rest tiny, ties at the cut among the tiny
    c = np.full(4096, 1e-3, np.float32); c[rng.choice(4096, 50, replace=False)] = 5.0; chunks.append(c)
    # boundary-threshold values next to 2s/3
    c = z.copy(); c[0] = 3.0; c[1:40] = 2.0; c[40:80] = np.nextafter(np.float32(2), np.float32(3))
    chunks.append(c)
    # huge and tiny normal magnitudes
    c = (rng.standard_normal(4096) * 1e37).astype(np.float32); chunks.append(c)
    c = (rng.standard_normal(4096) * 1e-37).astype(np.float32); chunks.append(c)
    return np.concatenate(chunks)


def test_tricky_chunks(orc):
    sl = require_gpu()
    rng = np.random.default_rng(123)
    d = _tricky_chunks(rng)
    for beta in (0.95, 1.0):
        ef = np.zeros_like(d)
        for rnd in range(3):
            ef = check_round(sl, orc, d, ef, beta, f"tricky beta={beta} round {rnd}")
    # negative-zero ef with -0 delta keeps acc = -0
    e = np.where(np.signbit(d), np.float32(-0.0), np.float32(0.0)).astype(np.float32)
    check_round(sl, orc, d, e, 0.95, "tricky signed-zero ef")


@pytest.mark.parametrize("beta", [0.0, 0.5, -0.75, 1.5, float(np.float32(1e-30))])
def test_other_decays(orc, beta):
    """Any finite decay: beta = 0 (no memory), a negative beta (products of
    either sign in the fma), beta > 1 and a tiny beta (beta * ef underflows to
    denormals or zero), each over three rounds on lognormal chunks."""
    sl = require_gpu()
    n = 64 * 4096
    ef = np.zeros(n, np.float32)
    for rnd in range(3):
        d = datagen.lognormal(n, datagen.SMALL_1M, 0, 40 + rnd).numpy()
        ef = check_round(sl, orc, d, ef, beta, f"beta={beta} round {rnd}")


def test_random_small_integer_chunks(orc):
    """Many chunks with values in a tiny integer set: every selection level
    and the index tie-break get exercised at scale."""
    sl = require_gpu()
    rng = np.random.default_rng(77)
    for span in (1, 2, 5, 50, 5000):
        d = rng.integers(-span, span + 1, 512 * 4096).astype(np.float32)
        ef = (rng.integers(-span, span + 1, d.size) * 0.5).astype(np.float32)
        check_round(sl, orc, d, ef, 0.95, f"int span {span}")


def test_edge_crossing_concatenation(orc):
    """Tensors concatenated so chunk boundaries fall inside tensors: the
    compressor only sees the flat buffer."""
    sl = require_gpu()
    sizes = datagen.edge_crossing_layout()
    parts = [datagen.lognormal(s + (-s) % 1024, datagen.DECODER_BLOCK, i, 0).numpy()[:s]
             for i, s in enumerate(sizes)]
    d = np.concatenate(parts).astype(np.float32)
    assert d.size % 4096 == 0
    check_round(sl, orc, d, np.zeros_like(d), 0.95, "edge crossing")


def test_determinism_and_delta_aliasing(orc):
    sl = require_gpu()
    n = 64 * 4096
    d = datagen.lognormal(n, datagen.SMALL_1M, 3, 0).numpy()
    e = datagen.lognormal(n, datagen.SMALL_1M, 4, 0).numpy() * np.float32(0.2)
    note("determinism: two identical calls")
    a = gpu_round(sl, d, e, 0.95)
    b = gpu_round(sl, d, e, 0.95)
    for x, y, w in zip(a, b, ("payload", "scales", "ef")):
        assert_bitwise(x, y, f"repeat {w}")
    # delta and ef the same buffer
    note("delta aliasing ef")
    t = torch.from_numpy(d.copy()).cuda()
    payload, scales = sl.compress(t, t, 0.95)
    torch.cuda.synchronize()
    op, os_, oe = orc.compress(d, d, beta=0.95)
    assert_bitwise(payload.cpu().numpy(), op, "aliased payload")
    assert_bitwise(t.cpu().numpy(), oe, "aliased ef")


def test_non_finite_chunks_stay_in_bounds(orc):
    """NaN and Inf inputs are outside the contract (their codes are
    unspecified), but they must not make the kernel write outside its chunk or
    loop without end.  Chunks holding NaN, +-Inf or a NaN error-feedback entry
    sit between finite chunks in one call.  The finite chunks must still match
    the oracle bit for bit, and guard regions around every output must be
    untouched, aggregated too."""
    sl = require_gpu()
    C = 12
    n = C * 4096
    G = 4096                                              # guard elements on each side
    rng = np.random.default_rng(99)
    d = (rng.standard_normal(n) * 0.3).astype(np.float32)
    e = (rng.standard_normal(n) * 0.05).astype(np.float32)
    bad = {2: "nan", 5: "inf", 6: "mixed", 9: "ef_nan"}
    for c, kind in bad.items():
        s = slice(c * 4096, (c + 1) * 4096)
        if kind == "nan":
            d[s][::7] = np.nan
        elif kind == "inf":
            d[s][::11] = np.inf
            d[s][5] = -np.inf
        elif kind == "mixed":
            d[s][:100] = np.nan
            d[s][100:164] = np.inf
        else:
            e[s][17] = np.nan
    dev = torch.device("cuda:0")
    sentinel = np.float32(-12345.5)
    dbuf = torch.full((n + 2 * G,), float(sentinel), dtype=torch.float32, device=dev)
    ebuf = torch.full((n + 2 * G,), float(sentinel), dtype=torch.float32, device=dev)
    pbuf = torch.full(((C + 2) * 112,), 0xA5, dtype=torch.uint8, device=dev)
    sbuf = torch.full((C + 2 * 16,), float(sentinel), dtype=torch.float32, device=dev)
    dbuf[G:G + n] = torch.from_numpy(d).to(dev)
    ebuf[G:G + n] = torch.from_numpy(e).to(dev)
    payload = pbuf[112:112 + C * 112].view(C, 112)
    scales = sbuf[16:16 + C]
    note("non-finite chunks: sl_compress")
    sl.sl_compress(dbuf[G:G + n], ebuf[G:G + n], 0.95, payload, scales)
    torch.cuda.synchronize()
    eb, pb, sb = ebuf.cpu().numpy(), pbuf.cpu().numpy(), sbuf.cpu().numpy()
    assert (eb[:G].view(np.uint32) == sentinel.view(np.uint32)).all()
    assert (eb[G + n:].view(np.uint32) == sentinel.view(np.uint32)).all()
    assert (pb[:112] == 0xA5).all() and (pb[112 + C * 112:] == 0xA5).all()
    assert (sb[:16].view(np.uint32) == sentinel.view(np.uint32)).all()
    assert (sb[16 + C:].view(np.uint32) == sentinel.view(np.uint32)).all()
    good = [c for c in range(C) if c not in bad]
    gd = np.concatenate([d[c * 4096:(c + 1) * 4096] for c in good])
    ge = np.concatenate([e[c * 4096:(c + 1) * 4096] for c in good])
    op, os_, oe = orc.compress(gd, ge, beta=0.95)
    gp = payload.cpu().numpy()[good]
    assert_bitwise(gp, op, "finite chunks' payload")
    assert_bitwise(scales.cpu().numpy()[good], os_, "finite chunks' scales")
    ef_new = eb[G:G + n]
    assert_bitwise(np.concatenate([ef_new[c * 4096:(c + 1) * 4096] for c in good]), oe, "finite chunks' ef")
    # The records of the non-finite chunks still have 12-bit fields, so an
    # aggregate of them stays inside its own chunks: guards around out intact.
    obuf = torch.full((n + 2 * G,), float(sentinel), dtype=torch.float32, device=dev)
    note("non-finite chunks: sl_aggregate of their records")
    sl.sl_aggregate([payload.contiguous()], [scales.contiguous()], obuf[G:G + n])
    torch.cuda.synchronize()
    ob = obuf.cpu().numpy()
    assert (ob[:G].view(np.uint32) == sentinel.view(np.uint32)).all()
    assert (ob[G + n:].view(np.uint32) == sentinel.view(np.uint32)).all()


def _structured_chunks(rng, n_chunks):
    """Chunks built to land the cut in every selection path: a small set of
    magnitudes (some a few ulps apart, some sharing the upper 13 or 23 key
    bits), each repeated at random indices spread over the whole chunk, over a
    quieter background, with random signs and signed zeros."""
    out = np.empty((n_chunks, 4096), np.float32)
    for c in range(n_chunks):
        base = np.float32(np.exp(rng.uniform(-20, 20)))
        bits = np.uint32(base.view(np.uint32))
        kind = c % 4
        if kind == 0:      # levels a few ulps apart: resolved by the last key bits
            offs = rng.integers(0, 8, 6)
        elif kind == 1:    # same exponent and 3 mantissa bits, differing in bits 19..10
            offs = rng.integers(0, 1 << 20, 6) & ~np.int64(0x3ff)
        elif kind == 2:    # differing anywhere in the low 20 bits
            offs = rng.integers(0, 1 << 20, 6)
        else:              # one repeated magnitude: index order decides
            offs = np.zeros(6, np.int64)
        levels = (bits + offs.astype(np.uint32)).view(np.float32)
        counts = rng.integers(0, 40, 6)
        bg_scale = np.float32(base * np.float32(rng.choice([0.0, 1e-3, 0.5, 0.99])))
        row = (rng.standard_normal(4096).astype(np.float32) * bg_scale).astype(np.float32)
        if rng.random() < 0.3:
            row[:] = bg_scale          # a flat background: ties below the levels
        pos = rng.permutation(4096)
        k = 0
        for lv, cnt in zip(levels, counts):
            row[pos[k:k + cnt]] = lv
            k += cnt
        row *= np.where(rng.random(4096) < 0.5, np.float32(-1), np.float32(1))
        row[rng.random(4096) < 0.01] = -0.0
        out[c] = row
    return out.reshape(-1)


def test_structured_selection_paths(orc):
    """2048 structured chunks over two rounds (beta 0.95, then beta 1 on the
    evolved ef), bitwise against the oracle."""
    sl = require_gpu()
    rng = np.random.default_rng(2024)
    d = _structured_chunks(rng, 2048)
    ef = np.zeros_like(d)
    ef = check_round(sl, orc, d, ef, 0.95, "structured round 0")
    check_round(sl, orc, _structured_chunks(rng, 2048), ef, 1.0, "structured round 1")
