"""Pins of the oracle to facts outside itself (CPU only).

Each test checks the oracle against something the pages print, a closed
form, a textbook or library routine, brute force, or an invariant of the
method -- never against a retyping of the oracle's own formula.  The
sections cited are those of "The inference core" page.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import workloads as W
from workloads import blob as B
from workloads.configs import Shape
from conftest import read_table, golden_constants

M64 = (1 << 64) - 1


def s64(v: int) -> int:
    v &= M64
    return v - (1 << 64) if v >> 63 else v


# --------------------------------------------------------------------------
# "The resumable state": the four run-account sizes the page prints

def test_pages_state_sizes_match_printed_values():
    rows = read_table("state_sizes.txt")
    assert len(rows) == 4
    for r in rows:
        cfg = tuple(int(v) for v in r[1:8])
        pb, mx, cp, size = (int(v) for v in r[8:12])
        assert O.pages_state_size(cfg, pb, mx) == size, r
        # the cache-positions rule: prompt bytes + max + 1, up to the context
        assert min(pb + mx + 1, cfg[6]) == cp


def test_ids_state_shares_the_pages_buffer_table():
    # The ids-in state differs from the page's account only in its first
    # buffers; from the activations on the two are the same table.
    cfg = (288, 768, 6, 6, 6, 32000, 256)
    L = O.state_layout(cfg, 10, 16)
    cp = 10 + 16 - 1
    assert L["cache_positions"] == cp
    assert L["ids"] == 128 and L["out"] == 128 + 40
    assert L["w1"] - L["x"] == 8 * 288 and L["up"] - L["gate"] == 8 * 768
    assert L["scores"] - L["logits"] == 8 * 32000
    assert L["keys"] - L["scores"] == 8 * cp
    assert L["values"] - L["keys"] == 4 * 6 * cp * 288
    assert L["total"] - L["values"] == 4 * 6 * cp * 288
    pages = O.pages_state_size(cfg, 0, cp - 1)  # cache positions = 0 + (cp-1) + 1
    tail_pages = pages - 256 - (128 + 0 + 8 + 4 * (cp - 1) + 128 * (cp - 1))
    assert L["total"] - L["x"] == tail_pages


# --------------------------------------------------------------------------
# "RMS normalization"

def test_isqrt_matches_math_isqrt():
    rng = np.random.default_rng(5)
    cases = list(range(0, 5000)) + [2**64 - 1, 2**63, 2**62, 2**32, 2**32 - 1]
    for k in [1, 2, 3, 255, 65535, 65536, 2**31 - 1, 2**31, 2**32 - 1]:
        cases += [k * k - 1, k * k, k * k + 1, k * k + 2 * k]
    cases += [int(v) for v in rng.integers(0, 2**63, 2000, dtype=np.uint64)]
    cases += [int(v) << 1 for v in rng.integers(0, 2**63, 500, dtype=np.uint64)]
    for n in cases:
        n &= M64
        assert O.isqrt(n) == math.isqrt(n), n


def test_rmsnorm_of_constant_vector_is_one():
    # mean(x^2) = x^2 for a constant vector, so x / rms(x) = sign(x): with
    # unit weights the output is exactly +-1.0 (2^16) for c >= 1.
    for d in (1, 7, 64, 4096):
        for c in (1, 2, 3, 100):
            for sign in (1, -1):
                x = np.full(d, sign * c * 65536, dtype=np.int64)
                w = np.full(d, 1 << 24, dtype=np.int32)
                assert np.all(O.rmsnorm(x, w) == sign * 65536), (d, c, sign)


def test_rmsnorm_epsilon_against_textbook():
    # y = x * w / sqrt(mean(x^2) + 1e-5) with the page's epsilon; at tiny
    # inputs the epsilon dominates, so a wrong epsilon fails.
    K = golden_constants()
    assert K["rms_epsilon_q32"] == round(1e-5 * 2**32)
    rng = np.random.default_rng(7)
    for scale in (1e-4, 1e-3, 3e-3, 1e-2, 0.5, 3.0):
        xr = rng.standard_normal(256) * scale
        x = np.rint(xr * 65536).astype(np.int64)
        gr = 1.0 + 0.05 * rng.standard_normal(256)
        w = np.rint(gr * 2**24).astype(np.int32)
        xq, wq = x / 65536.0, w / 2.0**24
        ref = xq * wq / np.sqrt(np.mean(xq * xq) + 1e-5)
        got = O.rmsnorm(x, w) / 65536.0
        # integer square root and two truncations: a few parts in rms, plus 2 ulp
        rms = math.sqrt(np.mean(xq * xq) + 1e-5) * 65536
        tol = np.abs(ref) * 2.0 / rms + 2.0 / 65536
        assert np.all(np.abs(got - ref) <= tol), scale


def test_rmsnorm_division_truncates_then_floors():
    # One element, weight 1.0: y = (x * 2^24 / rms) >> 8.  For x = -1 (Q16)
    # the quotient truncates to a small negative number and the shift
    # floors it to -1: a floor division would give the same here, so use a
    # case where truncation and floor differ before the shift.
    x = np.array([-3], dtype=np.int64)
    w = np.array([1 << 24], dtype=np.int32)
    rms = math.isqrt(9 // 1 + 42950)
    q = -((3 * (1 << 24)) // rms)          # truncation toward zero
    assert O.rmsnorm(x, w)[0] == q >> 8     # Python >> floors


# --------------------------------------------------------------------------
# "A matrix row"

def signed_dot(w, x):
    return sum((int(b) - 128) * int(v) for b, v in zip(w, x))


@pytest.mark.parametrize("n", [1, 7, 8, 9, 64, 172, 1000])
def test_row_equals_signed_dot_under_wrap(n):
    # The page: unsigned bytes times 64-bit words, corrected once by
    # 128 * sum, equal the signed dot product modulo 2^64.  Scale 2^24 shows
    # the low 40 bits of that dot and scale 1 its high 40 bits.
    rng = np.random.default_rng(n)
    for trial in range(4):
        w = rng.integers(0, 256, n, dtype=np.uint8)
        if trial == 0:
            x = rng.integers(-2**20, 2**20, n, dtype=np.int64)
        else:
            x = W.adversarial_row_inputs(1, n, 100 * n + trial)[0]
        dot = signed_dot(w, x)
        assert O.row(w, 1 << 24, x) == s64(dot << 24) >> 24
        assert O.row(w, 1, x) == s64(dot) >> 24
        if trial == 0:
            assert O.row(w, 1 << 24, x) == dot


def test_row_scale_zero_and_powers_of_two():
    rng = np.random.default_rng(1)
    w = rng.integers(0, 256, 300, dtype=np.uint8)
    x = rng.integers(-2**30, 2**30, 300, dtype=np.int64)
    dot = signed_dot(w, x)
    assert O.row(w, 0, x) == 0
    for k in range(0, 32):
        # y = floor(dot * 2^k / 2^24) while the product stays in range, and
        # the wrapped product beyond it
        want = (dot << k) >> 24 if abs(dot << k) < 2**63 else s64(dot << k) >> 24
        assert O.row(w, 1 << k, x) == want, k


def test_row_matches_scaled_dot_with_floor():
    rng = np.random.default_rng(2)
    for n in (16, 4096):
        w = rng.integers(0, 256, n, dtype=np.uint8)
        x = np.rint(rng.standard_normal(n) * 2 * 65536).astype(np.int64)
        for s in rng.integers(1 << 14, 1 << 18, 5):
            s = int(s)
            assert O.row(w, s, x) == (signed_dot(w, x) * s) // (1 << 24)


def test_rows_batch_is_rows_of_single_vectors():
    Wm, s, x = W.row_operands(37, 53, 5, 9)
    y = O.rows(Wm, s, x)
    for b in range(5):
        for r in (0, 1, 36):
            assert y[b, r] == O.row(Wm[r], int(s[r]), x[b])


def test_rows_threads_do_not_change_results():
    Wm, s, x = W.row_operands(257, 300, 3, 11)
    O.set_threads(1)
    y1 = O.rows(Wm, s, x)
    O.set_threads(4)
    y4 = O.rows(Wm, s, x)
    O.set_threads(1)
    assert np.array_equal(y1, y4)


def test_attention_threads_do_not_change_results():
    # The heads of a layer run on several threads when a turn covers them
    # whole; every state word (outputs, the scores buffer, the cursor's
    # largest score and sum) is the one-thread walk's, with grouped heads,
    # after cuts inside attention and at T > 0.
    shape = Shape(96, 160, 2, 8, 2, 300, 64)
    blob = B.build_blob(shape, 31)
    cfg = shape.as_tuple()
    for ids_n, mx, temp, seed in ((40, 6, 0, 3), (9, 20, 65536, 5)):
        ids = W.prompt_ids(shape.vocab, ids_n, 77, seed)
        outs = []
        for threads in (1, 6):
            O.set_threads(threads)
            e, st = O.init_state(cfg, ids, mx, temp, seed)
            assert e == 0
            # a turn of units that stops inside the first layer's attention
            # (sequential from there), then whole positions
            assert O.turn_units(blob, st, 4 + 96 * 3 + 3 * 4) == 0
            assert O.turn(blob, st, 3) == 0
            outs.append(st.copy())
            assert O.run_to_end(blob, st) == 0
            outs.append(st.copy())
        O.set_threads(1)
        assert np.array_equal(outs[0], outs[2]) and np.array_equal(outs[1], outs[3])


# --------------------------------------------------------------------------
# Phase 8, rotary

def test_rotation_special_angles():
    rng = np.random.default_rng(3)
    one = 1 << 24
    for _ in range(200):
        a, b = (int(v) for v in rng.integers(-2**38, 2**38, 2))
        assert O.rotate(a, b, one, 0) == (a, b)          # 0 degrees
        assert O.rotate(a, b, 0, one) == (-b, a)         # 90 degrees
        assert O.rotate(a, b, -one, 0) == (-a, -b)       # 180 degrees
        assert O.rotate(a, b, 0, -one) == (b, -a)        # 270 degrees


def test_rotation_matches_real_rotation():
    rng = np.random.default_rng(4)
    for _ in range(500):
        th = rng.uniform(-math.pi, math.pi)
        c, s = round(math.cos(th) * 2**24), round(math.sin(th) * 2**24)
        a, b = (int(v) for v in rng.integers(-2**24, 2**24, 2))
        ra = (a * c - b * s) / 2**24
        rb = (a * s + b * c) / 2**24
        ga, gb = O.rotate(a, b, c, s)
        assert abs(ga - ra) < 1.0 and abs(gb - rb) < 1.0


# --------------------------------------------------------------------------
# "Lookup tables"

def test_exp_index_rules():
    K = golden_constants()
    cap = K["exp_index_cap"]
    assert O.exp_index(0) == 0 and O.exp_index(255) == 0 and O.exp_index(256) == 1
    assert O.exp_index(cap * 256 - 1) == cap - 1
    assert O.exp_index(cap * 256) == cap
    assert O.exp_index(2**40) == cap and O.exp_index(2**64 - 1) == cap
    # a step of 1/256 in a Q16 difference: index = floor(d_real * 256)
    rng = np.random.default_rng(6)
    for d in rng.integers(0, 16 * 65536, 2000):
        assert O.exp_index(int(d)) == math.floor(Fraction(int(d), 65536) * 256)


def test_silu_index_and_edges_with_identity_table():
    # With TAB[i] = i the table lookup shows its index: for -16 < x < 16 it
    # is floor((x + 16) * 128), a step of 1/128 from -16.
    tab = np.arange(4097, dtype=np.int32)
    lim = golden_constants()["silu_limit_q16"]
    assert lim == 16 * 65536
    assert O.silu(lim, tab) == lim and O.silu(lim + 12345, tab) == lim + 12345
    assert O.silu(2**62, tab) == 2**62
    assert O.silu(-lim, tab) == 0 and O.silu(-2**62, tab) == 0
    assert O.silu(-lim + 1, tab) == 0 and O.silu(lim - 1, tab) == 4095
    rng = np.random.default_rng(8)
    for x in rng.integers(-lim + 1, lim, 3000):
        x = int(x)
        assert O.silu(x, tab) == math.floor((Fraction(x, 65536) + 16) * 128)


def test_silu_with_real_table_approximates_silu():
    tab = B.silu_table()
    rng = np.random.default_rng(9)
    for xr in rng.uniform(-20, 20, 2000):
        x = int(round(xr * 65536))
        got = O.silu(x, tab) / 65536.0
        xq = x / 65536.0
        want = xq / (1 + math.exp(-xq)) if abs(xq) < 16 else (xq if xq >= 16 else 0.0)
        # the table steps by 1/128 and SiLU's slope is below 1.1
        assert abs(got - want) <= 1.1 / 128 + 2 / 65536, xr


# --------------------------------------------------------------------------
# "Attention, stage by stage"

def test_attention_single_position_returns_value():
    exp_tab = B.exp_table()
    assert exp_tab[0] == 1 << 30
    rng = np.random.default_rng(10)
    for head in (2, 16, 128):
        q = rng.integers(-2**20, 2**20, head).astype(np.int64)
        K = rng.integers(-2**20, 2**20, (1, head)).astype(np.int32)
        V = rng.integers(-2**31, 2**31, (1, head), dtype=np.int64).astype(np.int32)
        out, p, m, ssum = O.attention_head(q, K, V, 2**24 // 4, exp_tab)
        assert p[0] == 1 << 24 and ssum == 1 << 30
        assert np.array_equal(out, V[0].astype(np.int64))


def test_attention_equal_scores_give_uniform_weights():
    exp_tab = B.exp_table()
    rng = np.random.default_rng(11)
    for n in (2, 3, 7, 100, 1000):
        q = rng.integers(-2**18, 2**18, 16).astype(np.int64)
        K = np.tile(rng.integers(-2**18, 2**18, 16).astype(np.int32), (n, 1))
        c = rng.integers(-2**20, 2**20, 16)
        V = np.tile(c.astype(np.int32), (n, 1))
        out, p, m, ssum = O.attention_head(q, K, V, 4194304, exp_tab)
        assert ssum == n << 30
        assert np.all(p == (1 << 24) // n)
        assert np.array_equal(out, (n * ((1 << 24) // n) * c.astype(object)) // (1 << 24))


def test_attention_score_scaling_and_max():
    # Scores: (((q . k) >> 16) * inv) >> 24; with inv = 2^24 / sqrt(head)
    # that is the textbook q . k / sqrt(head) in Q16, floored twice.
    exp_tab = B.exp_table()
    rng = np.random.default_rng(12)
    head = 64
    inv = round(2**24 / math.sqrt(head))
    assert inv == 2097152
    q = rng.integers(-2**17, 2**17, head).astype(np.int64)
    K = rng.integers(-2**17, 2**17, (40, head)).astype(np.int32)
    V = rng.integers(-2**17, 2**17, (40, head)).astype(np.int32)
    _, _, m, _ = O.attention_head(q, K, V, inv, exp_tab)
    dots = [int(np.dot(q.astype(object), K[j].astype(object))) for j in range(40)]
    scores = [((d >> 16) * inv) >> 24 for d in dots]
    assert m == max(scores)
    # and it is within two ulp of the real scaled dot
    real = max(d / 65536.0 / math.sqrt(head) for d in dots)
    assert abs(m - real) <= 2


def test_attention_matches_softmax_attention():
    exp_tab = B.exp_table()
    rng = np.random.default_rng(13)
    for head, n in ((16, 5), (64, 33), (128, 200)):
        inv = round(2**24 / math.sqrt(head))
        qr = rng.standard_normal(head)
        Kr = rng.standard_normal((n, head))
        Vr = rng.standard_normal((n, head))
        q = np.rint(qr * 65536).astype(np.int64)
        K = np.rint(Kr * 65536).astype(np.int32)
        V = np.rint(Vr * 65536).astype(np.int32)
        out, p, m, ssum = O.attention_head(q, K, V, inv, exp_tab)
        sc = (K / 65536.0) @ (q / 65536.0) / math.sqrt(head)
        pr = np.exp(sc - sc.max())
        pr /= pr.sum()
        ref = pr @ (V / 65536.0)
        # probabilities: the table steps by 1/256 in the score difference
        assert np.all(np.abs(p / 2**24 - pr) <= pr * (1 / 256.0 + 1e-3) + 2**-23)
        assert np.all(np.abs(out / 65536.0 - ref) <= 0.01 * np.abs(V / 65536.0).max() + 1e-4)


def test_attention_saturated_differences_use_last_entry():
    # Differences of 16 or more all read entry 4,096.
    exp_tab = np.arange(4097, dtype=np.uint32) + 1  # strictly positive, shows the index
    head = 2
    q = np.array([65536, 0], dtype=np.int64)
    inv = 1 << 24
    K = np.array([[0, 0], [-17 * 65536, 0], [-16 * 65536, 0], [-255, 0]], dtype=np.int32)
    V = np.zeros((4, 2), dtype=np.int32)
    _, p, m, ssum = O.attention_head(q, K, V, inv, exp_tab)
    # scores (Q16): 0, -17.0, -16.0, -255/65536 -> floor -> -1 (one ulp)
    e = [exp_tab[0], exp_tab[4096], exp_tab[4096], exp_tab[0]]
    assert ssum == sum(int(v) for v in e)
    assert m == 0


# --------------------------------------------------------------------------
# "Sampling"

def test_xorshift_multiplier_is_the_printed_constant():
    M = golden_constants()["xorshift_multiplier"]
    rng = np.random.default_rng(14)
    for st in rng.integers(1, 2**63, 50, dtype=np.uint64):
        new, out = O.xorshift64s(int(st))
        if new % 2 == 1:
            # the multiplier is out / new modulo 2^64 (new is invertible)
            assert (out * pow(new, -1, 1 << 64)) % (1 << 64) == M


def _gf2_matmul(A, Bm):
    # rows as 64-bit masks: (A*B) row i = xor of B rows j where A[i] has bit j
    out = []
    for a in A:
        acc = 0
        j = 0
        while a:
            if a & 1:
                acc ^= Bm[j]
            a >>= 1
            j += 1
        out.append(acc)
    return out


def _gf2_pow(A, e):
    R = [1 << i for i in range(64)]
    while e:
        if e & 1:
            R = _gf2_matmul(R, A)
        A = _gf2_matmul(A, A)
        e >>= 1
    return R


def test_xorshift_state_map_has_full_period():
    # Marsaglia's xorshift generators are the GF(2)-linear maps T of maximal
    # period 2^64 - 1: T^(2^64-1) = I and T^((2^64-1)/p) != I for each prime
    # p dividing 2^64 - 1.  The map is read off the oracle one bit at a time.
    cols = [O.xorshift64s(1 << i)[0] for i in range(64)]
    # T as row masks: bit j of row i = bit i of T(e_j)
    T = [sum(((cols[j] >> i) & 1) << j for j in range(64)) for i in range(64)]
    I = [1 << i for i in range(64)]
    order = (1 << 64) - 1
    assert _gf2_pow(T, order) == I
    for p in (3, 5, 17, 257, 641, 65537, 6700417):
        assert _gf2_pow(T, order // p) != I, p


def test_seed_zero_starts_at_golden_ratio_constant():
    # 0x9E3779B97F4A7C15 is floor(2^64 / phi) = floor(2^63 (sqrt 5 - 1)).
    K = golden_constants()
    phi_frac = (math.isqrt(5 << 128) - (1 << 64)) // 2
    assert phi_frac == K["seed_zero_state"]
    cfg = (64, 172, 1, 4, 4, 512, 32)
    e, st = O.init_state(cfg, [5, 6], 4, 0, 0)
    assert e == 0 and O.state_info(st)[1]["generator"] == K["seed_zero_state"]
    e, st = O.init_state(cfg, [5, 6], 4, 0, 77)
    assert O.state_info(st)[1]["generator"] == 77


def test_greedy_is_first_argmax():
    rng = np.random.default_rng(15)
    exp_tab = B.exp_table()
    for _ in range(50):
        lg = rng.integers(-5, 5, 300).astype(np.int64)  # many ties
        tok, g = O.sample(lg, 0, exp_tab, 123)
        assert tok == int(np.argmax(lg)) and g == 123


def test_draw_walk_is_inverse_cdf():
    # At temperature 1.0 (2^16) the sum pass reads the same entries as
    # attention; the walk then picks the entry whose prefix-sum interval holds
    # the draw: searchsorted over the cumulative sum.
    rng = np.random.default_rng(16)
    exp_tab = B.exp_table()
    M = golden_constants()["xorshift_multiplier"]
    for trial in range(40):
        V = int(rng.integers(2, 500))
        lg = rng.integers(-20 * 65536, 20 * 65536, V).astype(np.int64)
        seed = int(rng.integers(1, 2**63))
        tok, g = O.sample(lg, 65536, exp_tab, seed)
        new, _ = O.xorshift64s(seed)
        assert g == new
        m = int(lg.max())
        e = np.array([exp_tab[O.exp_index(m - int(v))] for v in lg], dtype=np.uint64)
        cs = np.cumsum(e)
        r = ((new * M) % (1 << 64)) % int(cs[-1])
        assert tok == int(np.searchsorted(cs, r, side="right"))


def test_temperature_sampling_frequencies():
    # Over many seeds the draw follows the weights e_i / sum.
    exp_tab = B.exp_table()
    lg = np.array([0, -65536, -2 * 65536, -30 * 65536], dtype=np.int64)
    counts = np.zeros(4)
    n = 20000
    for s in range(1, n + 1):
        tok, _ = O.sample(lg, 65536, exp_tab, s * 0x9E3779B97F4A7C15 % (1 << 64))
        counts[tok] += 1
    want = np.exp(-np.arange(4.0) * np.array([1, 1, 1, 1]))
    want[3] = math.exp(-16)
    want /= want.sum()
    assert np.all(np.abs(counts / n - want) < 0.015)


def test_xorshift_worked_steps_from_seed_one():
    # States and the first draw worked by hand from the three printed shift
    # steps ("Sampling"); the mirrored order of the shifts is also a
    # full-period map, so only worked values tell the two apart.
    g = {r[0]: int(r[1], 0) for r in read_table("xorshift_seed1.txt")}
    s1, d1 = O.xorshift64s(1)
    assert s1 == g["state_after_1"] and d1 == g["draw_1"]
    assert s1 != g["mirrored_state_after_1"]
    s2, _ = O.xorshift64s(s1)
    assert s2 == g["state_after_2"]
    # the sampler advances the generator by exactly this map at T > 0
    tok, gen = O.sample(np.array([0, -1], dtype=np.int64), 65536, B.exp_table(), 1)
    assert gen == g["state_after_1"]


def _one_hot_exp_table():
    # Entry 0 is 1 and every other entry 0: a logit whose difference indexes
    # entry 0 can be drawn, any other never.
    t = np.zeros(4097, dtype=np.uint32)
    t[0] = 1
    return t


@pytest.mark.parametrize("temp_q16, d_last0, d_first1", [
    (131072, 511, 512),    # T = 2.0: floor(d / 2) >> 8 is 0 up to d = 511
    (32768, 127, 128),     # T = 0.5: (2 d) >> 8 is 0 up to d = 127
    (65536, 255, 256),     # T = 1.0: the score-difference rule itself
    (1048576, 4095, 4096), # T = 16 (the largest): floor(d / 16) >> 8
])
def test_temperature_divides_the_difference(temp_q16, d_last0, d_first1):
    # "Sampling": the sum and draw passes take the largest logit minus each
    # logit, divide it by the temperature (both at 16 fractional bits) and
    # index the exponential table like a score difference.  With a table of
    # a single nonzero entry, the lower logit is drawn (about half the
    # seeds) exactly when its quotient indexes entry 0, and never otherwise.
    tab = _one_hot_exp_table()
    seeds = [(s * 0x9E3779B97F4A7C15) % (1 << 64) or 1 for s in range(1, 65)]
    for d, drawn in ((d_last0, True), (d_first1, False)):
        lg = np.array([0, -d], dtype=np.int64)
        toks = [O.sample(lg, temp_q16, tab, s)[0] for s in seeds]
        assert (1 in toks) == drawn, (temp_q16, d)
        if drawn:
            assert 16 < sum(toks) < 48  # the two weights are equal


@pytest.mark.parametrize("temp_q16", [131072, 32768])
def test_temperature_sampling_frequencies_away_from_one(temp_q16):
    # Away from T = 1 the draw follows exp(-d / T): logits one unit apart
    # give weights exp(-i / T) (entry round(256 i / T) of the table).
    exp_tab = B.exp_table()
    T = temp_q16 / 65536.0
    lg = np.array([0, -65536, -2 * 65536, -3 * 65536], dtype=np.int64)
    counts = np.zeros(4)
    n = 20000
    for s in range(1, n + 1):
        tok, _ = O.sample(lg, temp_q16, exp_tab, s * 0x9E3779B97F4A7C15 % (1 << 64))
        counts[tok] += 1
    want = np.exp(-np.arange(4.0) / T)
    want /= want.sum()
    assert np.all(np.abs(counts / n - want) < 0.015), (counts / n, want)


# --------------------------------------------------------------------------
# The artifact, the state and "Core errors"

def tiny_setup(shape=None, seed=1000):
    shape = shape or W.TINY.shape
    bl = B.build_blob(shape, seed)
    return shape, bl


def test_blob_check_accepts_and_rejects():
    shape, bl = tiny_setup()
    assert O.blob_check(bl) == (0, shape.as_tuple())
    bad = bl.copy(); bad[0] = ord("X")
    assert O.blob_check(bad)[0] == 2
    bad = bl.copy(); bad[8:12] = np.frombuffer(np.uint32(63).tobytes(), np.uint8)  # dim % heads
    assert O.blob_check(bad)[0] == 1
    lay = B.plan(shape)
    bad = bl.copy(); bad[lay.offsets["exp"]:lay.offsets["exp"] + 4] = 0    # EXP[0] = 0
    assert O.blob_check(bad)[0] == 2
    assert O.blob_check(bl[: lay.sections[-1][0] + 10].copy())[0] == 5      # truncated
    bad = bl.copy(); bad[40] += 1                                            # matrix count
    assert O.blob_check(bad)[0] == 2
    bad = bl.copy(); d0 = lay.offsets["desc"]; bad[d0 + 8] += 1              # rows
    assert O.blob_check(bad)[0] == 2
    bad = bl.copy(); bad[d0 + 32 * 2] = bad[d0 + 32]                         # duplicate kind
    bad[d0 + 32 * 2 + 4] = bad[d0 + 32 + 4]
    assert O.blob_check(bad)[0] == 2
    # a section length shorter than its matrix
    bad = bl.copy()
    o = B.SECTION_TABLE + 16 * 3 + 8
    bad[o:o + 8] = np.frombuffer(np.uint64(100).tobytes(), np.uint8)
    assert O.blob_check(bad)[0] == 5


def test_init_state_errors():
    cfg = W.TINY.shape.as_tuple()
    ctx = cfg[6]
    assert O.init_state(cfg, [5] * 4, 0)[0] == 6                     # max 0
    assert O.init_state(cfg, [5] * 4, ctx + 1)[0] == 6               # max > context
    assert O.init_state(cfg, [], 4)[0] == 6                          # no ids
    assert O.init_state(cfg, [512], 4)[0] == 6                       # id >= vocab
    assert O.init_state(cfg, [5], 4, 16 * 65536 + 1)[0] == 6         # temperature > 16
    assert O.init_state(cfg, [5], 4, 16 * 65536)[0] == 0
    assert O.init_state(cfg, [5] * 16, 17)[0] == 0                   # 16 + 17 - 1 = 32
    assert O.init_state(cfg, [5] * 16, 18)[0] == 7                   # 33 > 32
    assert O.init_state((0,) + cfg[1:], [5], 4)[0] == 1
    n = O.state_size(cfg, 3, 4)
    assert O.state_size(cfg, 3, 0) == 2**64 - 1
    assert O.init_state(cfg, [5] * 3, 4, state=O.aligned_zeros(n + 8))[0] == 4
    buf = O.aligned_zeros(n + 8)[1:n + 1]
    assert O.init_state(cfg, [5] * 3, 4, state=buf)[0] == 3           # misaligned


def test_turn_state_errors():
    shape, bl = tiny_setup()
    cfg = shape.as_tuple()
    e, st = O.init_state(cfg, [5, 6, 7], 2)
    bad = st.copy(); bad[0] = 0
    assert O.turn(bl, bad, 1) == 3
    assert O.turn(bl, st, 10) == 0
    assert O.state_info(st)[1]["complete"] == 1
    assert O.turn(bl, st, 1) == 3                                   # complete
    bad = bl.copy(); bad[0] = 0
    e, st = O.init_state(cfg, [5, 6, 7], 2)
    assert O.turn(bad, st, 1) == 2


def fit_failure_blob(shape, kind, seed=1000):
    """An artifact whose key or value rows overflow 32 bits at position 0."""
    bl = B.build_blob(shape, seed)
    w, s = B.matrix_view(bl, shape, kind, 0)
    w[:] = 255
    s[:] = 2**32 - 1
    return bl


@pytest.mark.parametrize("kind,phase", [(B.KIND_K, 6), (B.KIND_V, 7)])
def test_cache_fit_check_fails_with_arithmetic(kind, phase):
    shape = W.TINY.shape
    bl = fit_failure_blob(shape, kind)
    e, st = O.init_state(shape.as_tuple(), [5, 6, 7], 4)
    assert O.turn(bl, st, 4) == 8
    info = O.state_info(st)[1]
    assert (info["error"], info["phase"], info["layer"], info["position"]) == (8, phase, 0, 0)
    assert O.turn(bl, st, 1) == 3


def test_rotary_fit_check_fails_at_phase_8():
    # Keys that fit 32 bits before the rotation but not after it: key rows of
    # +-(2^31 - 1) turned by 45 degrees.
    shape = Shape(8, 16, 1, 1, 1, 16, 4)
    cos, sin = B.rope_tables(shape)
    c45 = round(2**24 * math.sqrt(0.5))
    cos[0, :] = c45
    sin[0, :] = c45
    bl = B.build_blob(shape, 5, tables={"cos": cos, "sin": sin, "norm": np.full(3 * 8, 1 << 24, np.int32)})
    w, s = B.matrix_view(bl, shape, B.KIND_K, 0)
    Wq, sq = B.matrix_view(bl, shape, B.KIND_EMBED, 0)
    # embedding: every element +1.0 exactly, so the normalized vector is all 1.0
    Wq[:] = 129
    sq[:] = 1 << 32 - 8  # (1 * 2^24) >> 8 = 2^16
    # key row 2j: +x, row 2j+1: -x with x just below 2^31
    w[0::2, :] = 255
    w[1::2, :] = 1
    s[:] = int((2**31 - 2**20) / (127 * 8) * 2**24 / 65536)
    e, st = O.init_state(shape.as_tuple(), [3], 2)
    assert O.turn(bl, st, 1) == 8
    info = O.state_info(st)[1]
    assert (info["phase"], info["layer"]) == (8, 0)


# --------------------------------------------------------------------------
# Whole-pass pins

def run_logits(shape, bl, ids, max_tokens, temp=0, seed=0):
    """Turn one position at a time; collect the logits at each generating
    position and the final state."""
    cfg = shape.as_tuple()
    e, st = O.init_state(cfg, ids, max_tokens, temp, seed)
    assert e == 0
    L = O.state_layout(cfg, len(ids), max_tokens)
    out = []
    while True:
        assert O.turn(bl, st, 1) == 0
        info = O.state_info(st)[1]
        if info["position"] >= len(ids):
            out.append(st[L["logits"]: L["logits"] + 8 * shape.vocab].view(np.int64).copy())
        if info["complete"]:
            break
    toks = st[L["out"]: L["out"] + 4 * max_tokens].view(np.uint32)[: info["generated"]].copy()
    return out, toks, st, L


@pytest.mark.parametrize("name", ["tiny", "gqa", "ragged"])
def test_whole_pass_tracks_float_forward(name):
    from float_model import FloatModel
    shape = W.SMALL_SHAPES[name]
    bl = B.build_blob(shape, 77)
    ids = W.prompt_ids(shape.vocab, 6, 5, 0)
    logits, toks, st, L = run_logits(shape, bl, ids, 8)
    fm = FloatModel(bl, shape)
    seq = list(ids) + list(toks)
    k = 0
    for t, tok in enumerate(seq[: len(ids) + len(toks) - 1]):
        lf, xf = fm.step(int(tok))
        if t >= len(ids) - 1:
            got = logits[k] / 65536.0
            k += 1
            assert np.abs(got - lf).max() < 0.05, (t, np.abs(got - lf).max())
            assert np.corrcoef(got, lf)[0, 1] > 0.999
    x = st[L["x"]: L["x"] + 8 * shape.dim].view(np.int64) / 65536.0
    assert np.abs(x - xf).max() < 0.05


def test_activations_stay_below_eight():
    shape = W.TINY.shape
    bl = B.build_blob(shape, 1000)
    ids = W.prompt_ids(shape.vocab, 16, 2000, 0)
    logits, toks, st, L = run_logits(shape, bl, ids, 16)
    assert len(toks) == 16
    x = st[L["x"]: L["x"] + 8 * shape.dim].view(np.int64)
    assert np.abs(x).max() < 8 * 65536


def test_incremental_equals_recompute():
    # Prefix runs (ids + the tokens generated so far, one token each) give the
    # same tokens as the one run that keeps its cache: the cache holds what a
    # recomputation would.
    shape = W.SMALL_SHAPES["gqa"]
    bl = B.build_blob(shape, 3)
    ids = W.prompt_ids(shape.vocab, 5, 9, 0)
    _, toks, _, _ = run_logits(shape, bl, ids, 6)
    seq = list(ids)
    for t in toks:
        _, tk, _, _ = run_logits(shape, bl, seq, 1)
        assert tk[0] == t
        seq.append(int(t))


def test_gqa_equals_mha_with_repeated_heads():
    # Head h reads key/value head h / (heads / kv_heads): a grouped model is
    # the same as the full-head model whose key and value rows repeat each
    # group's head.
    g = Shape(64, 96, 2, 8, 2, 100, 20)
    m = Shape(64, 96, 2, 8, 8, 100, 20)
    bg = B.build_blob(g, 21)
    bm = B.build_blob(m, 22)
    for l in range(2):
        for kind in B.LAYER_KINDS:
            wg, sg = B.matrix_view(bg, g, kind, l)
            wm, sm = B.matrix_view(bm, m, kind, l)
            if kind in (B.KIND_K, B.KIND_V):
                hs = g.head_size
                for h in range(8):
                    src = h // 4
                    wm[h * hs:(h + 1) * hs] = wg[src * hs:(src + 1) * hs]
                    sm[h * hs:(h + 1) * hs] = sg[src * hs:(src + 1) * hs]
            else:
                wm[:] = wg
                sm[:] = sg
    for kind in (B.KIND_EMBED, B.KIND_CLS):
        wm, sm = B.matrix_view(bm, m, kind)
        wg, sg = B.matrix_view(bg, g, kind)
        wm[:] = wg; sm[:] = sg
    lg, lm = B.plan(g), B.plan(m)
    for name in ("norm",):
        n = 4 * (2 * 2 + 1) * 64
        bm[lm.offsets[name]: lm.offsets[name] + n] = bg[lg.offsets[name]: lg.offsets[name] + n]
    ids = [7, 8, 9, 10]
    la, ta, _, _ = run_logits(g, bg, ids, 5)
    lb, tb, _, _ = run_logits(m, bm, ids, 5)
    assert np.array_equal(ta, tb)
    for a, b in zip(la, lb):
        assert np.array_equal(a, b)


def test_turn_cuts_do_not_change_results():
    shape = W.SMALL_SHAPES["ragged"]
    bl = B.build_blob(shape, 31)
    ids = W.prompt_ids(shape.vocab, 7, 3, 0)
    cfg = shape.as_tuple()
    e, a = O.init_state(cfg, ids, 9, 3 * 65536 // 2, 99)
    assert O.run_to_end(bl, a) == 0
    e, b = O.init_state(cfg, ids, 9, 3 * 65536 // 2, 99)
    for k in (1, 3, 2, 1, 4, 100):
        assert O.turn(bl, b, k) == 0
        if O.state_info(b)[1]["complete"]:
            break
    # only the turn counter differs
    ia, ib = O.state_info(a)[1], O.state_info(b)[1]
    assert ia["turns"] == 1 and ib["turns"] > 1
    a[80:88] = 0
    b[80:88] = 0
    assert np.array_equal(a, b)


# --------------------------------------------------------------------------
# Stopping between phases ("The resumable state")

H_PHASE, H_LAYER, H_ROW = 8, 12, 16


def set_cursor(st, phase, layer, row=0):
    st[H_PHASE:H_PHASE + 4] = np.frombuffer(np.uint32(phase).tobytes(), np.uint8)
    st[H_LAYER:H_LAYER + 4] = np.frombuffer(np.uint32(layer).tobytes(), np.uint8)
    st[H_ROW:H_ROW + 4] = np.frombuffer(np.uint32(row).tobytes(), np.uint8)


def test_each_phase_does_what_the_pages_list():
    # One phase per turn: the cursor walks the order of "The forward pass,
    # in order" (3, then 4-16 per layer, then 17-19 where a token is
    # generated), and each phase writes
    # the value of the building blocks pinned above, applied to the buffers
    # the previous phases left, into the buffer the pages name.
    shape = W.SMALL_SHAPES["gqa"]
    cfg = shape.as_tuple()
    bl = B.build_blob(shape, 41)
    lay = B.plan(shape)
    ids = W.prompt_ids(shape.vocab, 3, 4, 0)
    max_tokens = 3
    e, st = O.init_state(cfg, ids, max_tokens, 65536, 7)
    assert e == 0
    L = O.state_layout(cfg, len(ids), max_tokens)
    D, Hd, hs = shape.dim, shape.hidden, shape.head_size
    half, kvd, cp = hs // 2, shape.kv_dim, L["cache_positions"]

    def view(name, n, dt=np.int64):
        return st[L[name]: L[name] + np.dtype(dt).itemsize * n].view(dt)

    def table(name, n):
        return bl[lay.offsets[name]: lay.offsets[name] + 4 * n].view(np.int32)

    norm = table("norm", (2 * shape.layers + 1) * D).reshape(-1, D)
    cos = table("cos", shape.context * half).reshape(-1, half)
    sin = table("sin", shape.context * half).reshape(-1, half)
    exp_tab = table("exp", 4097).view(np.uint32)
    silu_tab = table("silu", 4097)
    keys = view("keys", shape.layers * shape.kv_heads * cp * hs, np.int32).reshape(
        shape.layers, shape.kv_heads, cp, hs)
    vals = view("values", shape.layers * shape.kv_heads * cp * hs, np.int32).reshape(
        shape.layers, shape.kv_heads, cp, hs)

    def mv(kind, layer, v):
        return O.rows(*B.matrix_view(bl, shape, kind, layer), v).reshape(-1)

    walked = []
    gen = O.state_info(st)[1]["generator"]
    while not O.state_info(st)[1]["complete"]:
        info = O.state_info(st)[1]
        p, l, t = info["phase"], info["layer"], info["position"]
        walked.append((p, l, t))
        x, w1, w2, w3 = (view(n, D).copy() for n in ("x", "w1", "w2", "w3"))
        gate, up = view("gate", Hd).copy(), view("up", Hd).copy()
        kc, vc = keys.copy(), vals.copy()
        assert O.turn_phases(bl, st, 1) == 0
        if p == 3:
            E, sE = B.matrix_view(bl, shape, B.KIND_EMBED)
            tok = info["token"]
            want = ((E[tok].astype(np.int64) - 128) * int(sE[tok])) >> 8
            assert np.array_equal(view("x", D), want)
        elif p in (4, 11, 17):
            xx = x + w1 if p == 11 else x
            assert np.array_equal(view("x", D), xx)
            k = 2 * shape.layers if p == 17 else 2 * l + (p == 11)
            assert np.array_equal(view("w1", D), O.rmsnorm(xx, norm[k]))
        elif p == 5:
            assert np.array_equal(view("w2", D), mv(B.KIND_Q, l, w1))
        elif p in (6, 7):
            kind, cache, before = (B.KIND_K, keys, kc) if p == 6 else (B.KIND_V, vals, vc)
            want = mv(kind, l, w1).reshape(shape.kv_heads, hs)
            assert np.array_equal(cache[l, :, t], want)
            before[l, :, t] = want
            assert np.array_equal(cache, before)
        elif p == 8:
            q = w2.copy()
            for h in range(shape.heads):
                for j in range(half):
                    i = h * hs + 2 * j
                    q[i], q[i + 1] = O.rotate(int(q[i]), int(q[i + 1]), int(cos[t, j]), int(sin[t, j]))
            assert np.array_equal(view("w2", D), q)
            for kh in range(shape.kv_heads):
                for j in range(half):
                    a, b = O.rotate(int(kc[l, kh, t, 2 * j]), int(kc[l, kh, t, 2 * j + 1]),
                                    int(cos[t, j]), int(sin[t, j]))
                    kc[l, kh, t, 2 * j:2 * j + 2] = (a, b)
            assert np.array_equal(keys, kc)
        elif p == 9:
            grp = shape.heads // shape.kv_heads
            for h in range(shape.heads):
                out = O.attention_head(w2[h * hs:(h + 1) * hs], keys[l, h // grp, :t + 1],
                                       vals[l, h // grp, :t + 1], B.inv_sqrt_head(shape), exp_tab)[0]
                assert np.array_equal(view("w3", D)[h * hs:(h + 1) * hs], out)
        elif p == 10:
            assert np.array_equal(view("w1", D), mv(B.KIND_O, l, w3))
        elif p in (12, 13):
            name, kind = ("gate", B.KIND_GATE) if p == 12 else ("up", B.KIND_UP)
            assert np.array_equal(view(name, Hd), mv(kind, l, w1))
        elif p == 14:
            want = [(O.silu(int(g), silu_tab) * int(u)) >> 16 for g, u in zip(gate, up)]
            assert np.array_equal(view("gate", Hd), np.array(want, np.int64))
        elif p == 15:
            assert np.array_equal(view("w1", D), mv(B.KIND_DOWN, l, gate))
        elif p == 16:
            assert np.array_equal(view("x", D), x + w1)
        elif p == 18:
            assert np.array_equal(view("logits", shape.vocab), mv(B.KIND_CLS, 0, w1))
        elif p == 19:
            tok, gen = O.sample(view("logits", shape.vocab), 65536, exp_tab, gen)
            after = O.state_info(st)[1]
            assert after["token"] == tok and after["generator"] == gen
            assert view("out", max_tokens, np.uint32)[info["generated"]] == tok
    per_layer = [(p, l) for l in range(shape.layers) for p in range(4, 17)]
    want = []
    for t in range(len(ids) + max_tokens - 1):
        want += [(3, 0, t)] + [(p, l, t) for p, l in per_layer]
        if t >= len(ids) - 1:
            want += [(17, 0, t), (18, 0, t), (19, 0, t)]
    # the run ends at the sampling of max_tokens tokens, or earlier at a
    # closing token
    assert walked == want[: len(walked)] and walked[-1][0] == 19
    assert len(walked) == len(want) or O.state_info(st)[1]["generated"] < max_tokens


def test_phase_cuts_do_not_change_results():
    # Turns that stop after any number of phases, mixed with turns of whole
    # positions, end in the state of one uninterrupted turn.
    shape = W.SMALL_SHAPES["ragged"]
    bl = B.build_blob(shape, 32)
    ids = W.prompt_ids(shape.vocab, 5, 6, 0)
    cfg = shape.as_tuple()
    e, a = O.init_state(cfg, ids, 7, 3 * 65536 // 2, 5)
    assert O.run_to_end(bl, a) == 0
    rng = np.random.default_rng(8)
    for trial in range(3):
        e, b = O.init_state(cfg, ids, 7, 3 * 65536 // 2, 5)
        while not O.state_info(b)[1]["complete"]:
            if rng.random() < 0.2:
                assert O.turn(bl, b, int(rng.integers(1, 3))) == 0
            else:
                assert O.turn_phases(bl, b, int(rng.integers(1, 40))) == 0
        a[80:88] = 0
        b[80:88] = 0
        assert np.array_equal(a, b)


def test_mid_position_cursor_checks():
    shape, bl = tiny_setup()
    cfg = shape.as_tuple()
    e, st = O.init_state(cfg, [5, 6, 7], 2)
    assert O.turn_phases(bl, st, 5) == 0
    info = O.state_info(st)[1]
    assert (info["phase"], info["layer"], info["position"]) == (8, 0, 0)
    for phase, layer in ((2, 0), (20, 0), (4, shape.layers), (3, 1), (17, 0), (21, 0)):
        bad = st.copy()
        set_cursor(bad, phase, layer)
        assert O.turn_phases(bl, bad, 1) == 3, (phase, layer)
    bad = st.copy()
    set_cursor(bad, 8, 0, row=1)                   # inside a phase
    assert O.turn_phases(bl, bad, 1) == 3
    assert O.turn_phases(bl, st, 0) == 0           # nothing to do
    assert O.state_info(st)[1]["phase"] == 8
    # a turn of positions finishes the one under way, then whole ones
    assert O.turn(bl, st, 1) == 0
    info = O.state_info(st)[1]
    assert (info["phase"], info["layer"], info["position"]) == (3, 0, 1)


H_STAGE, H_INDEX, H_PASS = 120, 124, 100
H_MAXSCORE, H_CHOSEN, H_SUM, H_REMAINDER, H_GENERATOR = 88, 96, 104, 112, 72


def u32(st, off):
    return int(st[off:off + 4].view(np.uint32)[0])


def u64(st, off):
    return int(st[off:off + 8].view(np.uint64)[0])


def i64(st, off):
    return int(st[off:off + 8].view(np.int64)[0])


def test_unit_cuts_do_not_change_results():
    # Turns that stop after any number of units of work (inside matrices,
    # attention stages and sampling passes), mixed with turns of phases and
    # of positions, end in the state of one uninterrupted turn.
    shape = W.SMALL_SHAPES["gqa"]
    bl = B.build_blob(shape, 33)
    ids = W.prompt_ids(shape.vocab, 5, 7, 0)
    cfg = shape.as_tuple()
    e, a = O.init_state(cfg, ids, 6, 65536, 9)
    assert O.run_to_end(bl, a) == 0
    rng = np.random.default_rng(10)
    for trial in range(3):
        e, b = O.init_state(cfg, ids, 6, 65536, 9)
        while not O.state_info(b)[1]["complete"]:
            u = rng.random()
            if u < 0.1:
                assert O.turn(bl, b, 1) == 0
            elif u < 0.2:
                assert O.turn_phases(bl, b, int(rng.integers(1, 5))) == 0
            else:
                assert O.turn_units(bl, b, int(rng.integers(1, [3, 40, 400][trial]))) == 0
        a[80:88] = 0
        b[80:88] = 0
        assert np.array_equal(a, b)


def test_attention_cursor_holds_each_stage():
    # One unit at a time through phase 9: the cursor's head, stage and index
    # walk heads, stages 0-3 and their units in order; the scores buffer and
    # the header hold each stage's values (scores and their maximum,
    # exponentials and their sum, probabilities), and the outputs so far are
    # those of the pinned whole-head routine.
    shape = W.SMALL_SHAPES["gqa"]
    cfg = shape.as_tuple()
    bl = B.build_blob(shape, 34)
    lay = B.plan(shape)
    ids = W.prompt_ids(shape.vocab, 6, 8, 0)
    e, st = O.init_state(cfg, ids, 2)
    L = O.state_layout(cfg, len(ids), 2)
    while True:                       # position 4, layer 1, phase 9
        i = O.state_info(st)[1]
        if (i["position"], i["layer"], i["phase"]) == (4, 1, 9):
            break
        assert O.turn_phases(bl, st, 1) == 0
    hs, cp, npos = shape.head_size, L["cache_positions"], 5
    exp_tab = bl[lay.offsets["exp"]: lay.offsets["exp"] + 4 * 4097].view(np.uint32)
    keys = st[L["keys"]: L["keys"] + 4 * shape.layers * shape.kv_heads * cp * hs].view(
        np.int32).reshape(shape.layers, shape.kv_heads, cp, hs)
    vals = st[L["values"]: L["values"] + 4 * shape.layers * shape.kv_heads * cp * hs].view(
        np.int32).reshape(shape.layers, shape.kv_heads, cp, hs)
    q = st[L["w2"]: L["w2"] + 8 * shape.dim].view(np.int64).copy()
    grp = shape.heads // shape.kv_heads
    want = [O.attention_head(q[h * hs:(h + 1) * hs], keys[1, h // grp, :npos].copy(),
                             vals[1, h // grp, :npos].copy(), B.inv_sqrt_head(shape), exp_tab)
            for h in range(shape.heads)]
    scores = lambda: st[L["scores"]: L["scores"] + 8 * npos].view(np.int64)
    w3 = lambda: st[L["w3"]: L["w3"] + 8 * shape.dim].view(np.int64)
    walk = []
    while O.state_info(st)[1]["phase"] == 9:
        h, sg, ix = u32(st, H_ROW), u32(st, H_STAGE), u32(st, H_INDEX)
        walk.append((h, sg, ix))
        out, p, m, ssum = want[h]
        if sg == 1 and ix > 0:
            assert u64(st, H_SUM) == int(scores()[:ix].sum())
        if sg >= 1:
            assert i64(st, H_MAXSCORE) == m
        if sg >= 2:
            assert u64(st, H_SUM) == ssum
        if sg == 3:
            assert np.array_equal(scores(), p)
            assert np.array_equal(w3()[h * hs: h * hs + ix], out[:ix])
        assert O.turn_units(bl, st, 1) == 0
    assert walk == [(h, sg, ix) for h in range(shape.heads) for sg in range(4)
                    for ix in range(npos if sg < 3 else hs)]
    # the phase's end: every head's output; the last head's maximum and sum
    for h in range(shape.heads):
        assert np.array_equal(w3()[h * hs:(h + 1) * hs], want[h][0])
    assert (i64(st, H_MAXSCORE), u64(st, H_SUM)) == (want[-1][2], want[-1][3])
    assert (u32(st, H_ROW), u32(st, H_STAGE), u32(st, H_INDEX)) == (0, 0, 0)


@pytest.mark.parametrize("temp", [0, 65536 * 3 // 4])
def test_sampling_cursor_holds_each_pass(temp):
    # One vocabulary entry at a time through phase 19: the maximum pass keeps
    # the running maximum and the first index that reached it; above
    # temperature zero the sum pass follows, the generator advances once
    # when it ends and the draw starts from xorshift64* modulo the sum; the
    # token is the pinned sampler's.
    shape = W.SMALL_SHAPES["gqa"]
    cfg = shape.as_tuple()
    bl = B.build_blob(shape, 35)
    lay = B.plan(shape)
    exp_tab = bl[lay.offsets["exp"]: lay.offsets["exp"] + 4 * 4097].view(np.uint32)
    ids = W.prompt_ids(shape.vocab, 3, 9, 0)
    e, st = O.init_state(cfg, ids, 3, temp, 77)
    L = O.state_layout(cfg, len(ids), 3)
    while O.state_info(st)[1]["phase"] != 19:
        assert O.turn_phases(bl, st, 1) == 0
    logits = st[L["logits"]: L["logits"] + 8 * shape.vocab].view(np.int64).copy()
    gen0 = u64(st, H_GENERATOR)
    want_tok, want_gen = O.sample(logits, temp, exp_tab, gen0)
    V = shape.vocab
    seen = []
    while O.state_info(st)[1]["phase"] == 19:
        ps, row = u32(st, H_PASS), u32(st, H_ROW)
        seen.append((ps, row))
        if ps == 0 and row > 0:
            assert i64(st, H_MAXSCORE) == logits[:row].max()
            assert u32(st, H_CHOSEN) == int(np.argmax(logits[:row]))
        if ps >= 1:
            assert u32(st, H_CHOSEN) == int(np.argmax(logits))
        if ps == 2 and row == 0:
            g, x = O.xorshift64s(gen0)
            assert u64(st, H_GENERATOR) == g
            assert u64(st, H_REMAINDER) == x % u64(st, H_SUM)
        assert O.turn_units(bl, st, 1) == 0
    passes = [(0, r) for r in range(V)]
    if temp:
        passes += [(1, r) for r in range(V)] + [(2, r) for r in range(want_tok + 1)]
    assert seen == passes
    assert u32(st, H_CHOSEN) == want_tok and O.state_info(st)[1]["token"] == want_tok
    assert u64(st, H_GENERATOR) == want_gen
    assert (u32(st, H_PASS), u32(st, H_ROW)) == (0, 0)


def test_matrix_cursor_holds_rows_done():
    # Inside a matrix phase the cursor's row counts the rows done; those rows
    # of the output hold the pinned row routine's values and the rest are
    # untouched; key and value rows go straight into the cache.
    shape = W.SMALL_SHAPES["ragged"]
    cfg = shape.as_tuple()
    bl = B.build_blob(shape, 36)
    ids = W.prompt_ids(shape.vocab, 3, 10, 0)
    e, st = O.init_state(cfg, ids, 2)
    L = O.state_layout(cfg, len(ids), 2)
    cp, hs = L["cache_positions"], shape.head_size
    for phase, kind, name, n in ((5, B.KIND_Q, "w2", shape.dim), (6, B.KIND_K, None, shape.kv_dim),
                                 (12, B.KIND_GATE, "gate", shape.hidden)):
        while O.state_info(st)[1]["phase"] != phase:
            assert O.turn_phases(bl, st, 1) == 0
        w1 = st[L["w1"]: L["w1"] + 8 * shape.dim].view(np.int64).copy()
        want = O.rows(*B.matrix_view(bl, shape, kind, 0), w1).reshape(-1)
        w3 = st[L["w3"]: L["w3"] + 8 * shape.dim].copy()
        before = st.copy()
        k = n // 3 + 1
        assert O.turn_units(bl, st, k) == 0
        assert O.state_info(st)[1]["phase"] == phase and u32(st, H_ROW) == k
        if name:
            buf = st[L[name]: L[name] + 8 * n].view(np.int64)
            old = before[L[name]: L[name] + 8 * n].view(np.int64)
            assert np.array_equal(buf[:k], want[:k]) and np.array_equal(buf[k:], old[k:])
        else:
            t = O.state_info(st)[1]["position"]
            keys = st[L["keys"]: L["keys"] + 4 * shape.layers * shape.kv_heads * cp * hs].view(
                np.int32).reshape(shape.layers, shape.kv_heads, cp, hs)
            assert np.array_equal(keys[0, :, t].reshape(-1)[:k], want[:k])
            assert np.array_equal(st[L["w3"]: L["w3"] + 8 * shape.dim], w3)
        assert O.turn_units(bl, st, n - k) == 0
        assert O.state_info(st)[1]["phase"] == phase + 1 and u32(st, H_ROW) == 0


def test_sub_phase_cursor_checks():
    shape, bl = tiny_setup()
    cfg = shape.as_tuple()

    def at(phase, **f):
        e, st = O.init_state(cfg, [5, 6, 7], 2, f.pop("temp", 0))
        while O.state_info(st)[1]["phase"] != phase:
            assert O.turn_phases(bl, st, 1) == 0
        for off, v in f.items():
            o = {"row": H_ROW, "stage": H_STAGE, "index": H_INDEX, "pass_": H_PASS,
                 "sum": H_SUM}[off]
            w = np.uint64(v) if off == "sum" else np.uint32(v)
            st[o:o + w.nbytes] = np.frombuffer(w.tobytes(), np.uint8)
        return st
    assert O.turn_units(bl, at(5, row=63), 1) == 0                 # a row inside the matrix
    assert O.turn_units(bl, at(5, row=64), 1) == 3                 # past the rows
    assert O.turn_units(bl, at(4, row=1), 1) == 3                  # a vector phase has no rows
    assert O.turn_units(bl, at(9, row=3), 1) == 0
    assert O.turn_units(bl, at(9, row=4), 1) == 3                  # no head 4
    assert O.turn_units(bl, at(9, stage=4), 1) == 3
    assert O.turn_units(bl, at(9, stage=0, index=1), 1) == 3       # position 0: one unit
    assert O.turn_units(bl, at(9, stage=3, index=15, sum=1 << 30), 1) == 0   # a head's elements
    assert O.turn_units(bl, at(9, stage=2, sum=0), 1) == 3         # no sum to divide by
    assert O.turn_units(bl, at(9, stage=1, pass_=1), 1) == 3
    assert O.turn_units(bl, at(19, pass_=1), 1) == 3               # temperature zero
    assert O.turn_units(bl, at(19, pass_=1, temp=65536), 1) == 0
    assert O.turn_units(bl, at(19, pass_=3, temp=65536), 1) == 3
    assert O.turn_units(bl, at(19, row=512), 1) == 3               # past the vocabulary


def stop_token_blob(shape, seed=1000):
    """Every activation +127.0 from the embedding, no residual updates, and a
    classifier whose only nonzero row is the closing token's: token 2 wins."""
    bl = B.build_blob(shape, seed, tables={"norm": np.full((2 * shape.layers + 1) * shape.dim,
                                                           1 << 24, np.int32)})
    E, sE = B.matrix_view(bl, shape, B.KIND_EMBED)
    E[:] = 255
    sE[:] = 1 << 24
    for l in range(shape.layers):
        for kind in (B.KIND_O, B.KIND_DOWN):
            B.matrix_view(bl, shape, kind, l)[1][:] = 0
    w, s = B.matrix_view(bl, shape, B.KIND_CLS)
    s[:] = 0
    s[2] = 1
    w[2, :] = 255
    return bl


def test_stop_token_completes_the_run():
    # A classifier that always prefers token 2 (the closing token): the first
    # sampled token completes the run.
    shape = W.TINY.shape
    bl = stop_token_blob(shape)
    e, st = O.init_state(shape.as_tuple(), [10, 11], 5)
    assert O.run_to_end(bl, st) == 0
    info = O.state_info(st)[1]
    assert info["complete"] and info["generated"] == 1
