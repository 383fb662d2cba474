"""Plant one plausible mistake at a time in a copy of the oracle; some pin must fail.

The mistakes are applied to the oracle's own source text on the CPU and run in
a scratch module; the real oracle is untouched.
"""
import importlib
import os
import types

import pytest

import oracle_pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

ATTN_MUTANTS = {
    "gqa_modulo": ("g = h // G\n                s = scale", "g = h % Hkv\n                s = scale"),
    "causal_strict": ("kv_pos[None, :] <= q_pos[:, None]", "kv_pos[None, :] < q_pos[:, None]"),
    "causal_reversed": ("kv_pos[None, :] <= q_pos[:, None]", "kv_pos[None, :] >= q_pos[:, None]"),
    "pad_attended": ("ok &= (q_seg != PAD_SEGMENT_ID)[:, None]", "pass"),
    "segment_compare": ("q_seg[:, None] == kv_seg[None, :]", "q_seg[:, None] >= kv_seg[None, :]"),
    "scale_dropped": ("s = scale * (q[b, r, h, :] @ k[b, :, g, :].T)\n                if softcap is not None:\n                    s = softcap",
                      "s = (q[b, r, h, :] @ k[b, :, g, :].T)\n                if softcap is not None:\n                    s = softcap"),
    "k_v_swapped": ("@ k[b, :, g, :].T)\n                if softcap is not None:\n                    s = softcap",
                    "@ v[b, :, g, :].T)\n                if softcap is not None:\n                    s = softcap"),
    "cap_factor_dropped": ("s = softcap * np.tanh(s / softcap)", "s = np.tanh(s / softcap)"),
    "sink_every_chunk": ("sinks=sinks if t == 0 else None", "sinks=sinks"),
    "sink_ignored": ("if sinks is not None:\n                    s = np.concatenate",
                     "if False:\n                    s = np.concatenate"),
    "merge_sigmoid_sign": ("sig = 1.0 / (1.0 + np.exp(-x))", "sig = 1.0 / (1.0 + np.exp(x))"),
    "merge_softplus_dropped": ("new_lse = lse + softplus", "new_lse = np.maximum(lse, block_lse)"),
    "merge_is_first_ignored": ("new_out = np.where(first4, block_out, new_out)", "pass"),
    "lse_log2": ("m_safe + np.log(np.where", "m_safe + np.log2(np.where"),
    "normaliser_off": ("o[nz] = num[nz] / z[nz, None]", "o[nz] = num[nz] / (z[nz, None] + 1e-3)"),
    "dense_ignored": ("ok &= dense != 0", "pass"),
    "dense_inverted": ("ok &= dense != 0", "ok &= dense == 0"),
    "dense_col0_ignored": ("c0 = a if dense_col0 is None else dense_col0[c]\n            dense_c = np.asarray(dense)[:, c0:c0 + (e - a)]\n        o_c",
                           "c0 = a\n            dense_c = np.asarray(dense)[:, c0:c0 + (e - a)]\n        o_c"),
    "dense_from_first_column": ("c0 = a if dense_col0 is None else dense_col0[c]\n            dense_c = np.asarray(dense)[:, c0:c0 + (e - a)]\n        o_c",
                                "c0 = 0 if dense_col0 is None else dense_col0[c]\n            dense_c = np.asarray(dense)[:, c0:c0 + (e - a)]\n        o_c"),
    "bwd_delta_dropped": ("du = p * (dp - Drow[:, None])", "du = p * dp"),
    "bwd_cap_chain_dropped": ("ds = du * (1.0 - t * t) if softcap is not None else du", "ds = du"),
    "bwd_dk_scale_dropped": ("dk[b, :, g, :] += scale * (ds.T @ q[b, r, h, :])", "dk[b, :, g, :] += ds.T @ q[b, r, h, :]"),
    "bwd_dv_from_ds": ("dv[b, :, g, :] += p.T @ do", "dv[b, :, g, :] += ds.T @ do"),
    "bwd_gqa_overwrite": ("dv[b, :, g, :] += p.T @ do", "dv[b, :, g, :] = p.T @ do"),
    "bwd_sink_sign": ("dsinks[h] -= float(np.sum(ps * Drow))", "dsinks[h] += float(np.sum(ps * Drow))"),
    "bwd_sink_every_chunk": ("sinks=sinks if c == 0 else None, dense=dense_c, out=out, lse=lse)",
                             "sinks=sinks, dense=dense_c, out=out, lse=lse)"),
    "bwd_chunk_local_lse": ("dense=dense_c, out=out, lse=lse)", "dense=dense_c, out=None, lse=None)"),
    "dq_rows_delta_dropped": ("g_logit = prob * (g_prob - delta[:, None])", "g_logit = prob * g_prob"),
    "dq_rows_cap_chain_dropped": ("g_logit = g_logit * (1.0 - tanh_t ** 2)", "g_logit = g_logit"),
    "dq_rows_scale_dropped": ("grad[b, :, h, :] = scale * np.einsum", "grad[b, :, h, :] = np.einsum"),
    "dq_rows_gqa_modulo": ("kv_h = h // per_kv", "kv_h = h % Hkv"),
}
MASK_MUTANTS = {
    "no_empty_tiles": ("elif tile.any():", "elif True:"),
    "full_from_first_row": ("if tile.all():", "if tile[0].all():"),
    "col_idx_unsorted": ("col_idx[qb, :len(nz)] = nz", "col_idx[qb, :len(nz)] = nz[::-1]"),
    "bits_msb_first": ("np.uint32(1 << (j % 32))", "np.uint32(1 << (31 - j % 32))"),
    "bits_on_full_tiles": ("if cls[qb, kb] != TILE_PARTIAL:", "if cls[qb, kb] == TILE_EMPTY:"),
    "bits_word_index": ("bits[qb, kb, i, j // 32]", "bits[qb, kb, i, j % W]"),
}


def _load(path, name, old, new):
    src = open(path).read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType(name)
    mod.__file__ = path
    exec(compile(src.replace(old, new), path, "exec"), mod.__dict__)
    return mod


def _mutant(which, key):
    attn_path = os.path.join(ROOT, "oracle", "attention.py")
    mask_path = os.path.join(ROOT, "oracle", "blockmask.py")
    if which == "attn":
        a = _load(attn_path, "mut_attention", *ATTN_MUTANTS[key])
        m = importlib.import_module("oracle.blockmask")
    else:
        a = importlib.import_module("oracle.attention")
        m = _load(mask_path, "mut_blockmask", *MASK_MUTANTS[key])
    return types.SimpleNamespace(
        attention=a.attention, allowed=a.allowed, merge=a.merge, chunked=a.chunked,
        attention_bwd=a.attention_bwd, attention_dq=a.attention_dq, chunked_bwd=a.chunked_bwd,
        DEFAULT_MASK_VALUE=a.DEFAULT_MASK_VALUE, block_mask=m.block_mask, partial_bits=m.partial_bits,
        TILE_EMPTY=m.TILE_EMPTY, TILE_PARTIAL=m.TILE_PARTIAL, TILE_FULL=m.TILE_FULL)


def _caught(ora):
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(ora)
        except Exception:
            return pin.__name__
    return None


@pytest.mark.parametrize("key", sorted(ATTN_MUTANTS))
def test_attention_mutant_caught(key):
    assert _caught(_mutant("attn", key)) is not None, f"no pin catches mutant {key}"


@pytest.mark.parametrize("key", sorted(MASK_MUTANTS))
def test_blockmask_mutant_caught(key):
    assert _caught(_mutant("mask", key)) is not None, f"no pin catches mutant {key}"
