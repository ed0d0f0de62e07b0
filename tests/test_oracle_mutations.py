"""Plants plausible mistakes in the CPU oracle (on the CPU, in this process
only) and checks that at least one pin of test_oracle_pins fails for each.
This shows the pins constrain every step of the oracle."""
import numpy as np
import pytest

import oracle.nanospec_oracle as O
from tests.test_oracle_pins import PINS


def _topk_tie_desc(z, K):
    z = np.asarray(z, np.float64)
    K = min(int(K), len(z))
    order = np.lexsort((-np.arange(len(z)), -z))
    return order[:K]


def _topk_ascending(z, K):
    z = np.asarray(z, np.float64)
    K = min(int(K), len(z))
    return np.lexsort((np.arange(len(z)), z))[:K]


def _first_occ_keep_last(ids):
    ids = [int(x) for x in ids]
    out = []
    for i, x in enumerate(ids):
        if x not in ids[i + 1:]:
            out.append(x)
    return out


def _stream_update_dedup_against_S(S, tree, ver):
    out = list(S)
    for x in list(tree) + list(ver):
        if int(x) not in out:
            out.append(int(x))
    return out


def _stream_update_draft_raw(S, tree, ver):
    return list(S) + [int(x) for x in tree] + [int(x) for x in ver]


def _suffix_prefix(S, w):
    return list(S[:w])


def _suffix_off_by_one(S, w):
    return list(S[-(w - 1):]) if w > 1 and len(S) >= w else list(S)


def _active_recent_distinct(S, w):
    out = []
    for v in reversed(list(S)):
        if v not in out:
            out.append(v)
        if len(out) == w:
            break
    return np.array(sorted(out), dtype=np.int64)


def _bitmap_msb_first(I, V):
    words = np.zeros((V + 31) // 32, dtype=np.uint32)
    for v in I:
        words[int(v) >> 5] |= np.uint32(1) << np.uint32(31 - (int(v) & 31))
    return words


def _project_drop_last_col(h, R, dtype):
    return O.widen(h, dtype)[:, :-1] @ O.widen(R, dtype)[:, :-1].T


def _project_sign(h, R, dtype):
    return -(O.widen(h, dtype) @ O.widen(R, dtype).T)


def _widen_shift15(x, dtype):
    if dtype == "bf16":
        b = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(15)
        return b.view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def _widen_fp16_bias14(x, dtype):
    if dtype == "fp16":
        u = np.asarray(x, dtype=np.uint16).astype(np.int64)
        sign = np.where(u >> 15, -1.0, 1.0)
        e = (u >> 10) & 0x1F
        f = (u & 0x3FF).astype(np.float64)
        return sign * np.where(e == 0, f * 2.0 ** -24, (1024.0 + f) * np.exp2((e - 24).astype(np.float64)))
    return _widen_orig(x, dtype)


_widen_orig = O.widen


def _draft_topk_by_column(logits, I, k):
    logits = np.atleast_2d(np.asarray(logits, np.float64))
    I = np.asarray(I, np.int64)
    M = logits.shape[0]
    ids = np.full((M, k), -1, np.int64)
    vals = np.full((M, k), -np.inf)
    for m in range(M):
        order = np.lexsort((np.arange(len(I)), -logits[m]))[:k]
        ids[m, :len(order)] = I[order]
        vals[m, :len(order)] = logits[m, order]
    return ids, vals


def _draft_topk_no_map(logits, I, k):
    logits = np.atleast_2d(np.asarray(logits, np.float64))
    M = logits.shape[0]
    ids = np.full((M, k), -1, np.int64)
    vals = np.full((M, k), -np.inf)
    for m in range(M):
        order = np.lexsort((np.asarray(I), -logits[m]))[:k]
        ids[m, :len(order)] = order           # column index instead of global id
        vals[m, :len(order)] = logits[m, order]
    return ids, vals


def _init_stream_sorted_union(prompt, P):
    return [int(x) for x in prompt] + sorted(set(int(x) for x in np.asarray(P).reshape(-1)))


def _init_stream_rank_major(prompt, P):
    return [int(x) for x in prompt] + O.first_occurrence(np.asarray(P).T.reshape(-1))


def _gather_transposed_index(W, I):
    return np.asarray(W)[np.asarray(I)[::-1]]


def _packed_generic(slot_ids, I, *, order=sorted, pick_free=lambda f: f, free_leaving=True,
                    keep_slots=True, count_slots=False):
    old = np.asarray(slot_ids, dtype=np.int64)
    act = set(int(x) for x in np.asarray(I).reshape(-1))
    new = old.copy()
    if not keep_slots:
        new[:] = -1
    elif free_leaving:
        new[[s for s in range(len(new)) if new[s] >= 0 and int(new[s]) not in act]] = -1
    held = set(int(x) for x in new if x >= 0)
    ent = order(act - held)
    free = pick_free([s for s in range(len(new)) if new[s] < 0])[:len(ent)]
    new[free] = ent
    occ = [s for s in range(len(new)) if new[s] >= 0]
    n = len(occ) if count_slots else (occ[-1] + 1 if occ else 0)
    return new, np.array(free, dtype=np.int64), np.array(ent, dtype=np.int64), n


def _packed_highest_free(slot_ids, I):
    return _packed_generic(slot_ids, I, pick_free=lambda f: f[::-1])


def _packed_descending(slot_ids, I):
    return _packed_generic(slot_ids, I, order=lambda x: sorted(x, reverse=True))


def _packed_repack(slot_ids, I):
    return _packed_generic(slot_ids, I, keep_slots=False)


def _packed_keep_leaving(slot_ids, I):
    return _packed_generic(slot_ids, I, free_leaving=False)


def _packed_count_slots(slot_ids, I):
    return _packed_generic(slot_ids, I, count_slots=True)


def _packed_head_with_holes(h, W, slot_ids, n_slots, k, dtype):
    ids = np.asarray(slot_ids, dtype=np.int64)[:n_slots]
    return O.draft_topk(O.project(h, O.gather_rows(W, ids), dtype), ids, k)


class _SequenceCtxKeepsVerify(O.Sequence_):
    """Ctx-only read as 'no draft-tree ids', still appending C_ver."""

    def step(self, tree_ids, ver_ids):
        if self.mode == "ctx_only":
            self.S = O.stream_update(self.S, [], ver_ids)
        else:
            super().step(tree_ids, ver_ids)


class _SequenceExtKeepsPrompt(O.Sequence_):
    """Ext-only that forgets to drop the prompt."""

    def append_prompt(self, prompt):
        self.S = self.S + [int(x) for x in prompt]


def _log_softmax_raw(logits):
    return np.atleast_2d(np.asarray(logits, np.float64)).copy()


def _logprob_over_vocabulary(h, W, I, k, dtype, parent=None):
    """Normalises over every row of W instead of the active set."""
    dense = O.dense_logits(h, W, dtype)
    lse = np.log(np.exp(dense - dense.max(axis=1, keepdims=True)).sum(axis=1, keepdims=True)) + \
        dense.max(axis=1, keepdims=True)
    logp = O.project(h, O.gather_rows(W, I), dtype) - lse
    ids, vals = O.draft_topk(logp, I, k)
    if parent is not None:
        vals = vals + np.asarray(parent, np.float64)[:, None]
    return logp, ids, vals


def _logprob_no_parent(h, W, I, k, dtype, parent=None):
    logp = O.log_softmax_active(O.project(h, O.gather_rows(W, I), dtype))
    ids, vals = O.draft_topk(logp, I, k)
    return logp, ids, vals


def _select_ties_late(vals, ids, k):
    v = np.asarray(vals, np.float64).reshape(-1)
    live = np.flatnonzero(np.asarray(ids).reshape(-1) >= 0)
    order = live[np.lexsort((-live, -v[live]))][:k]
    out = np.full(k, -1, np.int64)
    out[:len(order)] = order
    return out


def _select_keeps_holes(vals, ids, k):
    v = np.asarray(vals, np.float64).reshape(-1)
    order = np.lexsort((np.arange(len(v)), -v))[:k]
    out = np.full(k, -1, np.int64)
    out[:len(order)] = order
    return out


MUTATIONS = [
    ("top_k", _topk_tie_desc),
    ("top_k", _topk_ascending),
    ("first_occurrence", _first_occ_keep_last),
    ("stream_update", _stream_update_dedup_against_S),
    ("stream_update", _stream_update_draft_raw),
    ("suffix", _suffix_prefix),
    ("suffix", _suffix_off_by_one),
    ("active_set", _active_recent_distinct),
    ("bitmap", _bitmap_msb_first),
    ("project", _project_drop_last_col),
    ("project", _project_sign),
    ("widen", _widen_shift15),
    ("widen", _widen_fp16_bias14),
    ("draft_topk", _draft_topk_by_column),
    ("draft_topk", _draft_topk_no_map),
    ("init_stream", _init_stream_sorted_union),
    ("init_stream", _init_stream_rank_major),
    ("gather_rows", _gather_transposed_index),
    ("packed_update", _packed_highest_free),
    ("packed_update", _packed_descending),
    ("packed_update", _packed_repack),
    ("packed_update", _packed_keep_leaving),
    ("packed_update", _packed_count_slots),
    ("packed_draft_head", _packed_head_with_holes),
    ("Sequence_", _SequenceCtxKeepsVerify),
    ("Sequence_", _SequenceExtKeepsPrompt),
    ("log_softmax_active", _log_softmax_raw),
    ("draft_logprob_topk", _logprob_over_vocabulary),
    ("draft_logprob_topk", _logprob_no_parent),
    ("select_best", _select_ties_late),
    ("select_best", _select_keeps_holes),
]


@pytest.mark.parametrize("attr,bad", MUTATIONS, ids=[f"{a}:{f.__name__}" for a, f in MUTATIONS])
def test_pins_catch_planted_mistake(monkeypatch, attr, bad):
    monkeypatch.setattr(O, attr, bad)
    caught = []
    for pin in PINS:
        try:
            pin(O)
        except Exception:   # an assertion or a shape error both count as caught
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {bad.__name__} in {attr}"
