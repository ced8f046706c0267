"""Pins of the rebase-on-evict comparison variant's oracle (CPU only).

Independent of the variant's own code path:
* with float64 storage and arithmetic the variant must equal the method's
  re-based attention and the brute force at absolute positions (the same number
  in exact arithmetic): this fixes the bookkeeping, both rotation directions and
  the shift amount e, across chunks, wraps and resets of the origin;
* the same exact variant gives the same stored keys whether tokens arrive one
  at a time (shifts of 1) or in chunks (shifts of e): R(-e) = R(-1)^e;
* bf16 rounding equals the nearest representable neighbour chosen directly
  (ties to even), over random and tie-case inputs;
* with no eviction a stored key is within half a bf16 ulp (plus float32 noise)
  of the float64 rotation of its input: one rounding only;
* in bf16 the stored keys drift away from the exact rotation as evictions
  accumulate (the hazard the variant exists to show), while keys that never
  lived through an eviction do not.
Planted mistakes (shift by +e instead of -e, shift by e - 1, rotating new tokens
by L1 instead of their own index) must fail the exactness pin.
"""

import numpy as np
import pytest

import oracle.attention as att
import oracle.rebase as rb
import oracle.rope as rope_mod


def _drive(stream, rng, steps, chunk_sizes, hkv, d, hist):
    """Append random tokens; keep the raw history (positions, k, v)."""
    for t in range(steps):
        n = chunk_sizes[t % len(chunk_sizes)]
        k = rng.standard_normal((n, hkv, d))
        v = rng.standard_normal((n, hkv, d))
        p0 = stream.led.next_pos
        stream.append(k, v)
        for j in range(n):
            hist.append((p0 + j, k[j], v[j]))


def _exact_checks(w, hkv, hq, d, chunk_sizes, steps, seed, p0=0, s0=None):
    rng = np.random.default_rng(seed)
    st = rb.RebaseStream(w, hkv, d, bf16=False, next_pos=p0, next_slot=s0, exact=True)
    hist = []
    worst, worst_bf = 0.0, 0.0
    for t in range(steps):
        _drive(st, rng, 1, [chunk_sizes[t % len(chunk_sizes)]], hkv, d, hist)
        c = min(chunk_sizes[t % len(chunk_sizes)], st.led.length)
        q = rng.standard_normal((c, hq, d))
        got = st.attention(q)
        pos = [h[0] for h in hist]
        live = [h for h in hist if h[0] >= st.led.origin]
        kw = np.array([h[1] for h in live])
        vw = np.array([h[2] for h in live])
        ref = att.chunk_rebased(q, kw, vw)
        nxt = st.led.next_pos
        bf = att.brute_force(q, np.arange(nxt - c, nxt), pos, [h[1] for h in hist], [h[2] for h in hist],
                             nxt, w)
        worst = max(worst, float(np.max(np.abs(got - ref))))
        worst_bf = max(worst_bf, float(np.max(np.abs(got - bf))))
    return worst, worst_bf


@pytest.mark.parametrize("w,hkv,hq,d,chunks,steps,p0", [
    (8, 2, 4, 8, [1], 40, 0),
    (12, 1, 2, 16, [3, 1, 5], 30, 1000),
    (7, 2, 2, 8, [7, 2], 20, 2**24 - 20),
    (16, 2, 4, 64, [4], 25, 123456),
])
def test_exact_variant_equals_method(w, hkv, hq, d, chunks, steps, p0):
    rebased, brute = _exact_checks(w, hkv, hq, d, chunks, steps, seed=w + d, p0=p0)
    assert rebased < 1e-11
    # brute force rotates at absolute positions: float64 angles there carry an
    # error of about position * 2^-52 radians
    assert brute < 1e-11 + 4e-16 * (p0 + steps * max(chunks))


def test_exact_shift_composition():
    """Chunks of 4 (shifts of 4) and single tokens (shifts of 1) store the same keys."""
    rng = np.random.default_rng(1)
    w, hkv, d = 10, 2, 16
    a = rb.RebaseStream(w, hkv, d, bf16=False, exact=True)
    b = rb.RebaseStream(w, hkv, d, bf16=False, exact=True)
    for _ in range(9):
        k = rng.standard_normal((4, hkv, d))
        v = rng.standard_normal((4, hkv, d))
        a.append(k, v)
        for j in range(4):
            b.append(k[j:j + 1], v[j:j + 1])
    ka, _ = a.window()
    kb, _ = b.window()
    assert np.max(np.abs(ka - kb)) < 1e-12


def _nearest_bf16_direct(x):
    """Nearest bf16 value by looking at the two candidates around x."""
    out = np.empty_like(x)
    for i, v in enumerate(x):
        u = int(np.float32(v).view(np.uint32))
        lo = np.uint32(u & 0xFFFF0000).view(np.float32)
        hi = np.uint32((u & 0xFFFF0000) + 0x10000).view(np.float32)
        dl, dh = abs(float(v) - float(lo)), abs(float(hi) - float(v))
        if dl < dh or (dl == dh and ((u >> 16) & 1) == 0):
            out[i] = lo
        else:
            out[i] = hi
    return out


def test_round_bf16_is_nearest_even():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(4000).astype(np.float32) * np.float32(3.0)
    # exact ties: finite values whose dropped 16 bits are exactly half an ulp,
    # with an even and an odd last kept bit
    base = (rng.standard_normal(200).astype(np.float32) * np.float32(7.0)).view(np.uint32)
    ties = (base & np.uint32(0xFFFE0000)) | np.uint32(0x8000)
    ties = np.concatenate([ties, ties | np.uint32(1 << 16)]).view(np.float32)
    for arr in (x, ties):
        got = rb.round_bf16(arr)
        assert np.array_equal(got.view(np.uint32), _nearest_bf16_direct(arr).view(np.uint32))


def test_coefficients_at_zero_and_float32():
    c, s = rb.coef_f32(0, 64)
    assert np.all(c == 1.0) and np.all(s == 0.0)
    c, s = rb.coef_f32(np.array([5, 77]), 128)
    ang = np.array([5.0, 77.0])[:, None] * rope_mod.inv_freq(128)
    assert c.dtype == np.float32 and np.array_equal(c, np.cos(ang).astype(np.float32))
    assert np.array_equal(s, np.sin(ang).astype(np.float32))


def test_no_eviction_one_rounding():
    rng = np.random.default_rng(3)
    w, hkv, d = 64, 2, 128
    st = rb.RebaseStream(w, hkv, d, bf16=True)
    raw = rb.round_bf16(rng.standard_normal((40, hkv, d)).astype(np.float32))
    st.append(raw[:25], raw[:25])
    st.append(raw[25:], raw[25:])
    kw, _ = st.window()
    exact = rope_mod.rotate(raw.astype(np.float64), np.broadcast_to(np.arange(40)[:, None], (40, hkv)))
    # one bf16 rounding (half an ulp, 2^-9 relative) plus float32 product/sum noise
    bound = np.abs(exact) * 2.0 ** -8 + 1e-6
    assert np.all(np.abs(kw - exact) <= bound)


def test_bf16_drift_accumulates():
    """Keys that lived through many evictions are further from the exact
    rotation than once-rounded keys: the error the method avoids."""
    rng = np.random.default_rng(4)
    w, hkv, d = 32, 1, 64
    st = rb.RebaseStream(w, hkv, d, bf16=True)
    hist = []
    for t in range(w * 8):
        k = rb.round_bf16(rng.standard_normal((1, hkv, d)).astype(np.float32))
        st.append(k, k)
        hist.append(k[0].astype(np.float64))
    kw, _ = st.window()
    exact = rope_mod.rotate(np.array(hist[-w:]), np.broadcast_to(np.arange(w)[:, None], (w, hkv)))
    err = np.abs(kw - exact).max(axis=(1, 2))         # per live key, oldest first
    old, new = err[:4].mean(), err[-4:].mean()        # ~w shifts vs ~0 shifts
    assert old > 2.0 * new
    assert err.max() > 2.0 ** -8                      # beyond one rounding of a unit value


@pytest.mark.parametrize("mutant", ["plus_e", "e_minus_1", "new_at_l1"])
def test_planted_variant_mistakes_fail(monkeypatch, mutant):
    orig_append = rb.RebaseStream.append

    def bad_append(self, k_new, v_new):
        k_new = np.asarray(k_new)
        n = k_new.shape[0]
        l0 = self.led.length
        slots, evicted = self.led.append(n)
        l1 = self.led.length
        e = l0 + n - l1
        if e > 0 and l1 > n:
            surv = [self.led.slot_of_live(r) for r in range(l1 - n)]
            shift = {"plus_e": -e, "e_minus_1": e - 1}.get(mutant, e)
            self.k[surv] = self._rot(self.k[surv], shift, conj=True) if shift >= 0 else \
                self._rot(self.k[surv], -shift, conj=False)
        for j, slot in enumerate(slots):
            r = l1 if mutant == "new_at_l1" else l1 - n + j
            self.k[slot] = self._rot(k_new[j], r, conj=False)
            self.v[slot] = v_new[j]
        return slots, evicted

    monkeypatch.setattr(rb.RebaseStream, "append", bad_append)
    assert _exact_checks(8, 2, 4, 8, [1, 3], 30, seed=9)[0] > 1e-6
    monkeypatch.setattr(rb.RebaseStream, "append", orig_append)
