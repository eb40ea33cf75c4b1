"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each mutant is a copy of an oracle module with one plausible slip (a dropped
term, a wrong sign or index, a transposed operand).  The copy is built from
the module's source text, swapped in for the pin tests, and at least one pin
must fail.  The real oracle is never modified.
"""
import inspect
import types

import pytest

import oracle.attention as real_attention
import oracle.kvcache as real_kvcache
import oracle.metadata as real_metadata
import oracle.schedule as real_schedule
from tests import test_oracle_attention as TA
from tests import test_oracle_kvcache as TK
from tests import test_oracle_metadata as TM
from tests import test_oracle_schedule as TS

ATTENTION_MUTANTS = [
    ("drop scale", "s = scale * (K @ qvec)", "s = (K @ qvec)"),
    ("lse without max", "return (w @ V) / l, m + math.log(l)", "return (w @ V) / l, math.log(l)"),
    ("unnormalised", "return (w @ V) / l, m + math.log(l)", "return (w @ V), m + math.log(l)"),
    ("transposed page/slot", "pool[page_row[t // page_size], t % page_size]",
     "pool[page_row[t % page_size], t // page_size]"),
    ("causal off by one", "max(0, int(L) - (q_per_req - 1 - i))", "max(0, int(L) - (q_per_req - i))"),
    ("causal reversed", "max(0, int(L) - (q_per_req - 1 - i))", "max(0, int(L) - i)"),
    ("head map modulo", "g = h // G\n                out[b, i, h]", "g = h % Hkv\n                out[b, i, h]"),
    ("split floor", "c = -(-n // num_splits) if n else 0", "c = max(1, n // num_splits) if n else 0"),
    ("split unclipped", "return min(p0 * page_size, L), min(p1 * page_size, L)",
     "return p0 * page_size, p1 * page_size"),
    ("merge linear weights", "w = np.exp(l2[r, :n] - m)", "w = l2[r, :n] - m + 1.0"),
    ("merge lse drops max", "lse[r] = m + math.log(tot)", "lse[r] = math.log(tot)"),
    ("softmax sign", "w = np.exp(s - m)", "w = np.exp(m - s)"),
    ("merge ignores split counts", "n = S if split_counts is None else int(split_counts[r // rows_per_req])",
     "n = S"),
    ("split ignores split counts", "Sb = S if split_counts is None else int(split_counts[b])", "Sb = S"),
]

METADATA_MUTANTS = [
    ("no clamp", "cache = [max(L, 0) for L in seq_lens]", "cache = [L for L in seq_lens]"),
    ("inclusive prefix", "cu_k = [0]\n    for L in cache:\n        cu_k.append(cu_k[-1] + L)",
     "cu_k = []\n    acc = 0\n    for L in cache:\n        acc += L\n        cu_k.append(acc)\n    cu_k.append(acc)"),
    ("floor page count", "n = -(-cache[b] // page_size)", "n = cache[b] // page_size"),
    ("slot column", "col = j * page_size", "col = j"),
    ("sentinel passthrough", "pt[b, j] = slot // page_size if slot >= 0 else 0", "pt[b, j] = slot // page_size"),
    ("rpi unchecked", "if r < 0 or r >= R:\n            continue", "if False:\n            continue"),
    ("strided off by one", "cu_q = [b * int(q_stride) for b in range(B + 1)]",
     "cu_q = [(b + 1) * int(q_stride) for b in range(B + 1)]"),
    ("order ascending", "key=lambda b: (-cache[b], b)", "key=lambda b: (cache[b], b)"),
    ("order ties reversed", "key=lambda b: (-cache[b], b)", "key=lambda b: (-cache[b], -b)"),
    ("swa untranslated", "swa = f2s[slot]", "swa = slot"),
    ("swa sentinel looked up", "return slot if slot >= 0 else None", "return slot"),
    ("swa negative mapped slot kept", "pt[b, j] = swa // page_size if swa >= 0 else 0",
     "pt[b, j] = swa // page_size"),
    ("swa mapping unbounded", "if slot is None or slot >= len(f2s):", "if slot is None:"),
    ("swa no tail", "for j in range(min(n, max_pages)):\n            slot = _first_slot",
     "for j in range(max_pages):\n            slot = _first_slot"),
]

SCHEDULE_MUTANTS = [
    ("bucket floor", "k = min(max(-(-L // bucket_tokens), 1), len(table)) - 1",
     "k = min(max(L // bucket_tokens, 1), len(table)) - 1"),
    ("bucket off by one", "k = min(max(-(-L // bucket_tokens), 1), len(table)) - 1",
     "k = min(max(-(-L // bucket_tokens), 0), len(table) - 1)"),
    ("no page clamp", "out.append(max(1, min(table[k], n, max_splits)))",
     "out.append(max(1, min(table[k], max_splits)))"),
    ("no max clamp", "out.append(max(1, min(table[k], n, max_splits)))",
     "out.append(max(1, min(table[k], n)))"),
    ("empty request gets no split", "out.append(max(1, min(table[k], n, max_splits)))",
     "out.append(max(0, min(table[k], n, max_splits)))"),
    ("order ascending", "key=lambda b: (-seq[b], b)", "key=lambda b: (seq[b], b)"),
    ("splits descending", "for s in range(int(split_counts[b])):",
     "for s in reversed(range(int(split_counts[b]))):"),
    ("item fields swapped", "items.append(b * ITEM_SHIFT + s)", "items.append(s * ITEM_SHIFT + b)"),
    ("padding not -1", "items + [-1] * (capacity - len(items))", "items + [0] * (capacity - len(items))"),
]


KVCACHE_MUTANTS = [
    ("int8 scale /128", "s = _fp16_scale(amax / _F32(127.0))", "s = _fp16_scale(amax / _F32(128.0))"),
    ("int8 floor", "q = np.rint(xf / s.astype(_F32)[..., None])", "q = np.floor(xf / s.astype(_F32)[..., None])"),
    ("no zero-scale guard", "return np.where(s == 0, np.float16(1.0), s)", "return s"),
    ("int4 scale /16", "s = _fp16_scale((mx - mn) / _F32(15.0))", "s = _fp16_scale((mx - mn) / _F32(16.0))"),
    ("int4 zero sign", "z = (np.clip(np.rint(-mn / sf), 0, 15)", "z = (np.clip(np.rint(mn / sf), 0, 15)"),
    ("int4 zero not added", "np.rint(g / sf[..., None]) + z.astype(_F32)[..., None]",
     "np.rint(g / sf[..., None])"),
    ("int4 nibble order", "(nib[..., 0::2] | (nib[..., 1::2] << 4))", "(nib[..., 1::2] | (nib[..., 0::2] << 4))"),
    ("int4 zero floor", "z = (np.clip(np.rint(-mn / sf), 0, 15)", "z = (np.clip(np.floor(-mn / sf), 0, 15)"),
    ("int4 zero keeps -0", "+ _F32(0.0)).astype(np.float16)", ").astype(np.float16)"),
    ("append page/offset swapped", "p, t = int(slot) // page_size, int(slot) % page_size",
     "t, p = int(slot) // page_size, int(slot) % page_size"),
    ("append past the pool", "if slot < 0 or slot >= P * page_size:", "if slot < 0:"),
    ("append sentinel", "if slot < 0 or slot >= P * page_size:", "if slot >= P * page_size:"),
]


def _mutant(module, old, new):
    src = inspect.getsource(module)
    assert src.count(old) >= 1, f"mutation site not found: {old!r}"
    src = src.replace(old, new)
    m = types.ModuleType(module.__name__ + "_mutant")
    m.__package__ = module.__package__
    exec(compile(src, module.__name__ + "_mutant", "exec"), m.__dict__)
    return m


def _attention_pins():
    g = TA._load_attention_golden()
    pins = [lambda c=c: TA.test_hand_derived_cases(c) for c in g["cases"]]
    pins += [TA.test_hand_derived_split_case,
             lambda: TA.test_matches_library_sdpa_on_dense_inputs(False, 1),
             lambda: TA.test_matches_library_sdpa_on_dense_inputs(True, 4),
             TA.test_length_one_gives_v0_exactly, TA.test_equal_scores_give_mean_of_v,
             TA.test_two_tokens_closed_form, TA.test_gqa_equals_mha_with_repeated_kv_heads,
             TA.test_mtp_query_equals_single_query_decode_on_shorter_cache,
             lambda: TA.test_split_then_merge_equals_unsplit(4),
             TA.test_split_ranges_partition_the_tokens,
             lambda: TS.test_per_request_splits_merge_to_the_unsplit_result(False, 1),
             lambda: TS.test_per_request_splits_merge_to_the_unsplit_result(True, 3)]
    return pins


def _metadata_pins():
    import oracle.metadata as OM
    pins = [lambda m=m, k=k, e=e: TM.test_hand_built_batch(m, k, e) for (m, k, e) in [
        (OM.Q_STRIDED, "cu_seqlens_q_strided", {}),
        (OM.Q_CUMSUM, "cu_seqlens_q_cumsum", {"q_in": "q_lens"}),
        (OM.Q_PRESET, "cu_seqlens_q_preset", {"q_in": "cu_q_preset"})]]
    pins += [TM.test_sentinels_never_produce_negative_or_out_of_range_ids,
             TM.test_swa_hand_built_batch, TM.test_swa_guards]
    pins += [lambda w=w: TM.test_swa_page_permutation_and_evictions(w) for w in TM.SWA_CASES]
    return pins


def _schedule_pins():
    return [TS.test_hand_built_schedule, TS.test_capacity_too_small_is_an_error,
            TS.test_constant_table_is_the_batch_wide_split]


def _kvcache_pins():
    pins = [lambda a=a: TK.test_int8_hand_rows(*a) for a in [
        ([0.0, 1.0, -1.0, 2.5, 127.0], 1.0, [0, 1, -1, 2, 127]),
        ([254.0, -3.0, 1.5, -0.5], 2.0, [127, -2, 1, 0]),
        ([0.0, 0.0, 0.0], 1.0, [0, 0, 0]),
        ([1e-9, -1e-9], 1.0, [0, 0])]]
    pins += [TK.test_int4_hand_row_rounding_zero_clamp_and_nibble_order,
             TK.test_int4_zero_point_zero_is_stored_as_plus_zero,
             TK.test_int4_all_equal_groups_decode_exactly, TK.test_int8_roundtrip_within_half_step,
             TK.test_int4_roundtrip_within_half_step,
             TK.test_append_writes_only_valid_slots_at_page_and_offset,
             TK.test_append_quantises_each_row_with_its_encoder]
    return pins


def _some_pin_fails(pins):
    for p in pins:
        try:
            p()
        except Exception:
            return True
    return False


def test_real_oracle_passes_every_pin():
    assert not _some_pin_fails(_attention_pins())
    assert not _some_pin_fails(_metadata_pins())
    assert not _some_pin_fails(_kvcache_pins())
    assert not _some_pin_fails(_schedule_pins())


@pytest.mark.parametrize("name,old,new", ATTENTION_MUTANTS, ids=[m[0] for m in ATTENTION_MUTANTS])
def test_attention_mutant_is_caught(monkeypatch, name, old, new):
    m = _mutant(real_attention, old, new)
    monkeypatch.setattr(TA, "OA", m)
    monkeypatch.setattr(TS, "OA", m)
    assert _some_pin_fails(_attention_pins()), f"no pin caught mutant '{name}'"


@pytest.mark.parametrize("name,old,new", METADATA_MUTANTS, ids=[m[0] for m in METADATA_MUTANTS])
def test_metadata_mutant_is_caught(monkeypatch, name, old, new):
    monkeypatch.setattr(TM, "OM", _mutant(real_metadata, old, new))
    assert _some_pin_fails(_metadata_pins()), f"no pin caught mutant '{name}'"


@pytest.mark.parametrize("name,old,new", KVCACHE_MUTANTS, ids=[m[0] for m in KVCACHE_MUTANTS])
def test_kvcache_mutant_is_caught(monkeypatch, name, old, new):
    monkeypatch.setattr(TK, "OK", _mutant(real_kvcache, old, new))
    assert _some_pin_fails(_kvcache_pins()), f"no pin caught mutant '{name}'"


@pytest.mark.parametrize("name,old,new", SCHEDULE_MUTANTS, ids=[m[0] for m in SCHEDULE_MUTANTS])
def test_schedule_mutant_is_caught(monkeypatch, name, old, new):
    monkeypatch.setattr(TS, "OS", _mutant(real_schedule, old, new))
    assert _some_pin_fails(_schedule_pins()), f"no pin caught mutant '{name}'"
