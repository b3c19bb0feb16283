"""Plant plausible mistakes in copies of the oracle (on the CPU) and require that the pins catch
each one.  This checks the pins, not the oracle: a pin set that a dropped term, a wrong sign or
index, or a transposed operand slips through would not be worth much."""

import importlib.util
import os
import sys
import types

import pytest

import oracle_pins as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _load_mutant(module: str, old: str, new: str, count: int = 1) -> types.ModuleType:
    path = os.path.join(ROOT, "oracle", module + ".py")
    src = open(path).read()
    assert src.count(old) >= count, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new)
    name = f"oracle_mutant_{module}_{abs(hash((old, new)))}"
    spec = importlib.util.spec_from_loader(name, loader=None)
    mod = importlib.util.module_from_spec(spec)
    mod.__dict__["__package__"] = "oracle"
    sys.modules[name] = mod
    exec(compile(src, path, "exec"), mod.__dict__)
    return mod


def _attention_pins(m):
    return [
        lambda: P.pin_bruteforce_decode(m.ref_attention),
        lambda: P.pin_bruteforce_prefill(m.ref_attention),
        lambda: P.pin_closed_forms(m.ref_attention),
        lambda: P.pin_gqa_head_map(m.ref_attention),
        lambda: P.pin_library_sdpa(m.ref_attention),
        lambda: P.pin_combine_invariance(m.ref_attention, m.ref_partial, m.ref_combine, trials=10),
        lambda: P.pin_partial_definition(m.ref_partial),
    ]


def _plan_pins(m):
    return [
        lambda: P.pin_worked_example(m.ref_plan, m.parse_map),
        lambda: P.pin_fill_closed_form(m.ref_plan, m.parse_map, trials=200),
        lambda: P.pin_budget_rule(m.ref_plan, m.parse_map, trials=100),
    ]


def _lpt_pins(m):
    return [
        lambda: P.pin_lpt_hand_example(m.ref_plan_lpt, m.parse_map),
        lambda: P.pin_lpt_equal_sizes_round_robin(m.ref_plan_lpt, m.parse_map),
        lambda: P.pin_lpt_coverage_and_balance(m.ref_plan_lpt, m.parse_map, trials=60),
    ]


def _rated_pins(m):
    return [
        lambda: P.pin_rated_hand_examples(m.ref_plan_rated, m.parse_map),
        lambda: P.pin_rated_equal_rates_are_weighted(m.ref_plan_rated, m.ref_plan_weighted, trials=40),
        lambda: P.pin_rated_contiguous_and_proportional(m.ref_plan_rated, m.parse_map, trials=60),
    ]


def _weighted_pins(m):
    return [
        lambda: P.pin_weighted_hand_examples(m.ref_plan_weighted, m.parse_map),
        lambda: P.pin_weighted_worked_example(m.ref_plan_weighted, m.parse_map),
        lambda: P.pin_weighted_contiguous_and_balanced(m.ref_plan_weighted, m.parse_map, trials=60),
    ]


def _store_pins(m):
    from oracle import fp8
    return [
        lambda: P.pin_round_bf16_library(m.round_bf16),
        lambda: P.pin_e4m3_round_library(m.e4m3_round, fp8.e4m3_table),
        lambda: P.pin_hadamard(m.hadamard),
        lambda: P.pin_rope(m.rope),
        lambda: P.pin_rms_norm_library(m.rms_norm),
        lambda: P.pin_store_kv_composition(m.ref_store_kv),
    ]


def _fp8_pins(m):
    return [
        lambda: P.pin_e4m3_library(m.e4m3_table),
        lambda: P.pin_e4m3_closed_forms(m.e4m3_value),
        lambda: P.pin_fp8_decode_library(m.ref_decode_fp8),
        lambda: P.pin_fp8_scale_laws(m.ref_decode_fp8),
    ]


def _caught(pins) -> bool:
    for pin in pins:
        try:
            pin()
        except Exception:
            return True
    return False


ATTENTION_MUTANTS = {
    "dropped scale": ("s = scale * (qg", "s = (qg"),
    "wrong sign in exponent": ("np.exp(s - np.where", "np.exp(s + np.where"),
    "causal bound off by one": ("first_row + np.arange(rows) + 1", "first_row + np.arange(rows)"),
    "mask keeps the diagonal+1": ("pos[None, :] < upto", "pos[None, :] <= upto"),
    "interleaved GQA head map": ("g * group:(g + 1) * group", "g::Hkv"),
    "keys used as values": ("p.reshape(-1, e - a) @ vg", "p.reshape(-1, e - a) @ kg"),
    "dropped first term of the sum": ("= p.sum(axis=2)", "= p[:, :, 1:].sum(axis=2)"),
    "combine without max shift weights": ("w = np.where(np.isfinite(ms), np.exp(ms - np.where(has, M, 0.0)[None]), 0.0)",
                                          "w = np.where(np.isfinite(ms), 1.0, 0.0)"),
    "combine divides by split count": ("Lsum = (w * ls).sum(axis=0)", "Lsum = (w * ls).sum(axis=0) * 0 + len(parts)"),
}

FP8_MUTANTS = {
    "exponent bias 8": ("E4M3_BIAS = 7", "E4M3_BIAS = 8"),
    "subnormals given the implicit one": ("return sign * mant * 2.0 ** (1 - E4M3_BIAS - E4M3_MANT_BITS)",
                                          "return sign * (1.0 + mant / 8.0) * 2.0 ** (1 - E4M3_BIAS)"),
    "sign bit ignored": ("sign = -1.0 if code & 0x80 else 1.0", "sign = 1.0"),
    "top code read as a number": ("if exp == 0xF and mant == 0x7:", "if False:"),
    "mantissa over 16": ("(1.0 + mant / 8.0)", "(1.0 + mant / 16.0)"),
    "values scaled with the key scale": ("v = dequantize_kv(v_codes[b], v_scale)", "v = dequantize_kv(v_codes[b], k_scale)"),
    "keys scaled with the value scale": ("k = dequantize_kv(k_codes[b], k_scale)", "k = dequantize_kv(k_codes[b], v_scale)"),
    "scale of the first head for all": ("vals * scale[None, :, None]", "vals * scale[0]"),
}

LPT_MUTANTS = {
    "ties to the highest worker": ("key=lambda i: (load[i], i))", "key=lambda i: (load[i], -i))"),
    "smallest tiles first": ("pieces.sort(key=lambda x: (-x[0], x[1], x[2]))", "pieces.sort(key=lambda x: (x[0], x[1], x[2]))"),
    "loads counted in tiles": ("load[w] += size", "load[w] += 1"),
    "most loaded worker": ("w = min(range(num_workers), key=lambda i: (load[i], i))",
                           "w = max(range(num_workers), key=lambda i: (load[i], -i))"),
    "runs not merged": ("if lst and lst[-1][0] == ui and lst[-1][2] == t - 1:", "if False:"),
}

WEIGHTED_MUTANTS = {
    "tile start instead of its midpoint": ("w = (num_workers * (2 * before + c)) // (2 * total_cost)",
                                           "w = (num_workers * (2 * before)) // (2 * total_cost)"),
    "split cost ignored": ("+ (split_cost if t == 0 else 0)))", "+ 0))"),
    "split cost on every tile": ("+ (split_cost if t == 0 else 0)))", "+ split_cost))"),
    "tiles counted, not tokens": ("stream.append((ui, t, min(tile, u.extent - t * tile) +",
                                  "stream.append((ui, t, tile +"),
    "worker index rounded up": ("w = (num_workers * (2 * before + c)) // (2 * total_cost)",
                                "w = min(num_workers - 1, -(-(num_workers * (2 * before + c)) // (2 * total_cost)))"),
}

RATED_MUTANTS = {
    "tile start instead of its midpoint": ("if 2 * C * share_start[v] <= R * (2 * P + c))",
                                           "if 2 * C * share_start[v] <= R * (2 * P))"),
    "share boundary owned by the earlier worker": ("if 2 * C * share_start[v] <= R * (2 * P + c))",
                                                   "if 2 * C * share_start[v] < R * (2 * P + c))"),
    "shares start one worker late": ("if 2 * C * share_start[v] <= R * (2 * P + c))",
                                     "if 2 * C * share_start[v + 1] <= R * (2 * P + c))"),
    "own rate instead of the running sum": ("share_start.append(share_start[-1] + r)", "share_start.append(r)"),
    "first worker instead of the last": ("w = max(v for v in range(num_workers) if 2 * C",
                                         "w = min(v for v in range(num_workers) if 2 * C"),
    "split cost ignored": ("tiles.append((ui, t, tokens + split_cost * (t == 0)))", "tiles.append((ui, t, tokens))"),
    "tiles counted, not tokens": ("tokens = min(tile, u.extent - t * tile)", "tokens = tile"),
    "rates reversed": ("    for r in rates:\n        share_start.append", "    for r in rates[::-1]:\n        share_start.append"),
}

STORE_MUTANTS = {
    "rope sign flipped": ("[x1 * c - x2 * s, x2 * c + x1 * s]", "[x1 * c + x2 * s, x2 * c - x1 * s]"),
    "rope frequency exponent": ("freq = theta ** (-2.0 * i / D)", "freq = theta ** (-1.0 * i / D)"),
    "rms norm without the gain": ("keepdims=True) + eps) * np.asarray(w, dtype=np.float64)", "keepdims=True) + eps)"),
    "rms norm over the sum": ("np.mean(x * x, axis=-1, keepdims=True)", "np.sum(x * x, axis=-1, keepdims=True)"),
    "hadamard without normalisation": ("hadamard_matrix(D).T / math.sqrt(D)", "hadamard_matrix(D).T"),
    "bf16 truncates": ("return np.round(np.ldexp(x, -step_exp))", "return np.trunc(np.ldexp(x, -step_exp))"),
    "e4m3 ties away": ("((hi - a == a - lo) & ((pos_codes[j] & 1) == 0))", "(hi - a == a - lo)"),
    "e4m3 drops the sign": ("return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)", "return code.astype(np.uint8)"),
    # the composition: which vector takes which step, gain and scale, in which order
    "rope applied to v": ("        k = rope(k, positions, theta)\n", "        k = rope(k, positions, theta)\n        v = rope(v, positions, theta)\n"),
    "hadamard applied to v": ("        k = hadamard(k)\n", "        k = hadamard(k)\n        v = hadamard(v)\n"),
    "v normalised with the key gain": ("return q_out, round_bf16(k), round_bf16(v)",
                                       "return q_out, round_bf16(k), round_bf16(v if k_norm_w is None else rms_norm(v, k_norm_w, eps))"),
    "hadamard skipped on q": ("        q = hadamard(q)\n", "        q = q\n"),
    "hadamard skipped on k": ("        k = hadamard(k)\n", "        k = k\n"),
    "rope skipped on k": ("        k = rope(k, positions, theta)\n", "        k = k\n"),
    "scales swapped": ("e4m3_round(k / ks), e4m3_round(v / vs)", "e4m3_round(k / vs), e4m3_round(v / ks)"),
    "v quantised with the key scale": ("e4m3_round(v / vs)", "e4m3_round(v / ks)"),
    "q takes the key gain": ("q = rms_norm(q, q_norm_w, eps)", "q = rms_norm(q, k_norm_w if k_norm_w is not None else q_norm_w, eps)"),
    "k takes the query gain": ("k = rms_norm(k, k_norm_w, eps)", "k = rms_norm(k, q_norm_w if q_norm_w is not None else k_norm_w, eps)"),
    "norm after rope": ("""    if q_norm_w is not None:
        q = rms_norm(q, q_norm_w, eps)
    if k_norm_w is not None:
        k = rms_norm(k, k_norm_w, eps)
    if theta > 0:
        q = rope(q, positions, theta)
        k = rope(k, positions, theta)
""", """    if theta > 0:
        q = rope(q, positions, theta)
        k = rope(k, positions, theta)
    if q_norm_w is not None:
        q = rms_norm(q, q_norm_w, eps)
    if k_norm_w is not None:
        k = rms_norm(k, k_norm_w, eps)
"""),
    "hadamard before rope": ("""    if theta > 0:
        q = rope(q, positions, theta)
        k = rope(k, positions, theta)
    if use_hadamard:
        q = hadamard(q)
        k = hadamard(k)
""", """    if use_hadamard:
        q = hadamard(q)
        k = hadamard(k)
    if theta > 0:
        q = rope(q, positions, theta)
        k = rope(k, positions, theta)
"""),
}

PLAN_MUTANTS = {
    "floor tile count": ("return ceil_div(extent, tile) if extent > 0 else 0", "return extent // tile"),
    "extra tiles to the last workers": ("base + (1 if w < rem else 0)", "base + (1 if w >= workers - rem else 0)"),
    "end not clipped to the request": ("min(u.extent, (t_last + 1) * tile)", "(t_last + 1) * tile"),
    "off-by-one segment start": ("Segment(u.b, u.qt, t_first * tile,", "Segment(u.b, u.qt, t_last * tile,"),
    "budget ignores the remainder": ("base, rem = divmod(total_tiles, workers)", "base, rem = -(-total_tiles // workers), 0"),
}


@pytest.mark.parametrize("name", sorted(ATTENTION_MUTANTS))
def test_attention_mutant_is_caught(name):
    old, new = ATTENTION_MUTANTS[name]
    m = _load_mutant("attention", old, new, count=1)
    assert _caught(_attention_pins(m)), f"no pin catches: {name}"


@pytest.mark.parametrize("name", sorted(PLAN_MUTANTS))
def test_plan_mutant_is_caught(name):
    old, new = PLAN_MUTANTS[name]
    m = _load_mutant("plan", old, new, count=1)
    assert _caught(_plan_pins(m)), f"no pin catches: {name}"


@pytest.mark.parametrize("name", sorted(LPT_MUTANTS))
def test_lpt_mutant_is_caught(name):
    old, new = LPT_MUTANTS[name]
    m = _load_mutant("plan", old, new, count=1)
    assert _caught(_lpt_pins(m)), f"no pin catches: {name}"


@pytest.mark.parametrize("name", sorted(WEIGHTED_MUTANTS))
def test_weighted_mutant_is_caught(name):
    old, new = WEIGHTED_MUTANTS[name]
    m = _load_mutant("plan", old, new, count=1)
    assert _caught(_weighted_pins(m)), f"no pin catches: {name}"


@pytest.mark.parametrize("name", sorted(RATED_MUTANTS))
def test_rated_mutant_is_caught(name):
    old, new = RATED_MUTANTS[name]
    m = _load_mutant("plan", old, new, count=1)
    assert _caught(_rated_pins(m)), f"no pin catches: {name}"


@pytest.mark.parametrize("name", sorted(STORE_MUTANTS))
def test_store_mutant_is_caught(name):
    old, new = STORE_MUTANTS[name]
    m = _load_mutant("store_kv", old, new, count=1)
    assert _caught(_store_pins(m)), f"no pin catches: {name}"


@pytest.mark.parametrize("name", sorted(FP8_MUTANTS))
def test_fp8_mutant_is_caught(name):
    old, new = FP8_MUTANTS[name]
    m = _load_mutant("fp8", old, new, count=1)
    assert _caught(_fp8_pins(m)), f"no pin catches: {name}"


def test_unmutated_oracle_passes_all_pins():
    import oracle.attention as A
    import oracle.fp8 as F
    import oracle.plan as Pl
    import oracle.store_kv as SK
    for pin in (_attention_pins(A) + _plan_pins(Pl) + _fp8_pins(F) + _lpt_pins(Pl) + _weighted_pins(Pl)
                + _rated_pins(Pl) + _store_pins(SK)):
        pin()
