"""Plant plausible mistakes in copies of the oracle and check the pins catch each.

Each mutant is the oracle's source text with one edit, loaded as a fresh
module on the CPU.  The pins of ``oracle_pins`` run against it; at least one
must fail.  This guards the pins themselves: a pin set that passes a dropped
term, a flipped sign, an off-by-one or a wrong index would not pin anything.
"""
import os
import types

import pytest

from . import oracle_pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "attention.py")

MUTANTS = {
    "drop_rope_term": ("s = s + qr.index_select(0, r) @ kr.T", "s = s + 0 * (qr.index_select(0, r) @ kr.T)"),
    "rope_unscaled": ("        s = scale * s\n", "        s = scale * s + (0 if qr is None else (1 - scale) * (qr.index_select(0, r) @ kr.T))\n"),
    "band_pre_sign": ("keep &= (i - j) <= int(pre_tokens)", "keep &= (j - i) <= int(pre_tokens)"),
    "band_pre_off_by_one": ("keep &= (i - j) <= int(pre_tokens)", "keep &= (i - j) < int(pre_tokens)"),
    "band_next_off_by_one": ("keep &= (j - i) <= int(next_tokens)", "keep &= (j - i) < int(next_tokens)"),
    "causal_strict": ("keep &= j <= i", "keep &= j < i"),
    "band_always_on": ("    if mask is not None or causal:\n        if pre_tokens", "    if True:\n        if pre_tokens"),
    "mask_polarity": ("keep &= mask.index_select(0, rows.to(torch.int64)) == 0", "keep &= mask.index_select(0, rows.to(torch.int64)) != 0"),
    "sink_not_in_denominator": ("            l = l + torch.exp(float(sink) - m_safe)", "            l = l + 0.0"),
    "sink_not_in_max": ("            m = torch.clamp(m, min=float(sink))", "            m = m"),
    "sink_scaled": ("m = torch.clamp(m, min=float(sink))", "m = torch.clamp(m, min=float(sink) * scale)"),
    "gqa_modulo": ("        g = h // group\n        return head_attention(qc", "        g = h % Nkv\n        return head_attention(qc"),
    "mask_head_broadcast": ("hh = h if mask.shape[1] > 1 else 0", "hh = 0"),
    "bsh_head_split": ("return x.reshape(b, s, heads, h // heads).permute(0, 2, 1, 3)", "return x.reshape(b, s, h // heads, heads).permute(0, 2, 1, 3)"),
    "empty_row_nan": ("o = torch.where((l > 0).view(-1, 1), num / torch.where(l > 0, l, torch.ones_like(l)).view(-1, 1),", "o = torch.where((l >= 0).view(-1, 1), num / l.view(-1, 1),"),
    "tnd_kv_uses_q_offsets": ("q0, q1, k0, k1 = cq[bi], cq[bi + 1], ck[bi], ck[bi + 1]", "q0, q1, k0, k1 = cq[bi], cq[bi + 1], cq[bi], cq[bi + 1]"),
    "no_neg_inf_guard": ("m_safe = torch.where(finite, m, torch.zeros_like(m))", "m_safe = m"),
    "pse_before_scale": ("        s = scale * s\n        if pse is not None:\n            s = s + pse.index_select(0, r).to(torch.float64)\n",
                         "        if pse is not None:\n            s = s + pse.index_select(0, r).to(torch.float64)\n        s = scale * s\n"),
    "pse_transposed": ("s = s + pse.index_select(0, r).to(torch.float64)", "s = s + pse.T.index_select(0, r).to(torch.float64)"),
    "pse_batch_broadcast": ("pse=pse[b if pse.shape[0] > 1 else 0, h]", "pse=pse[0, h]"),
    "pse_tnd_head_major": ("return pse.reshape(-1)[pse_off[bi]:pse_off[bi + 1]].view(N, lq, lk)[h]",
                           "return pse.reshape(-1)[pse_off[bi]:pse_off[bi + 1]].view(lq, N, lk)[:, h]"),
    "offset_sign": ("    i = il + int(q_start)\n", "    i = il - int(q_start)\n"),
    "offset_swapped": ("    j = jl + int(kv_start)\n", "    j = jl + int(q_start)\n"),
    "offset_on_mask": ("keep &= mask.index_select(0, rows.to(torch.int64)) == 0",
                       "keep &= mask.index_select(0, (rows.to(torch.int64) + int(q_start)) % mask.shape[0]) == 0"),
    "merge_drops_l": ("w = torch.where(torch.isfinite(ms), torch.exp(ms - m_safe) * ls, torch.zeros_like(ls))",
                      "w = torch.where(torch.isfinite(ms), torch.exp(ms - m_safe), torch.zeros_like(ls))"),
    "merge_sign": ("w = torch.where(torch.isfinite(ms), torch.exp(ms - m_safe) * ls, torch.zeros_like(ls))",
                   "w = torch.where(torch.isfinite(ms), torch.exp(m_safe - ms) * ls, torch.zeros_like(ls))"),
    "tnd_mask_outside_kept": ("    out = torch.ones(lq, lk, dtype=atten_mask.dtype)\n",
                              "    out = torch.zeros(lq, lk, dtype=atten_mask.dtype)\n"),
    "tnd_mask_outside_wraps": ("    out[:r, :c] = atten_mask[:r, :c]\n",
                               "    out[:r, :c] = atten_mask[:r, :c]\n    out[r:, :c] = atten_mask[:lq - r, :c] if lq - r <= atten_mask.shape[0] else out[r:, :c]\n"),
    "stats_layout_transposed": ("    if layout == \"TND\" and softmax_out_layout == \"same_as_input\":\n        x = x.transpose(0, 1)\n",
                                "    if layout == \"TND\" and softmax_out_layout == \"\":\n        x = x.transpose(0, 1)\n"),
}


def _load_mutant(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique in the oracle source"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


def _stats_layout_pin(orc):
    """expand_stats: "" -> [N, T, 8], "same_as_input" -> [T, N, 8]."""
    import torch
    x = torch.arange(6, dtype=torch.float64).view(2, 3)          # [N=2, T=3]
    a = orc.expand_stats(x, "TND", "")
    b = orc.expand_stats(x, "TND", "same_as_input")
    assert tuple(a.shape) == (2, 3, 8) and tuple(b.shape) == (3, 2, 8)
    assert float(a[1, 2, 5]) == 5.0 and float(b[2, 1, 7]) == 5.0


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    mod = _load_mutant(name)
    caught = []
    for pin in oracle_pins.ALL_PINS + [_stats_layout_pin]:
        try:
            pin(mod)
        except Exception as e:  # AssertionError, or the mutant crashing on a pin's input
            caught.append(f"{pin.__name__}: {type(e).__name__}")
            break
    assert caught, f"no pin detects mutant {name}"


def test_unmutated_oracle_passes_stats_layout():
    from oracle import attention
    _stats_layout_pin(attention)
