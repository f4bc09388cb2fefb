"""Planted mistakes, on the CPU, in copies of the oracle: each plausible slip
(a dropped term, a wrong sign or index, a transposed operand, a wrong
frequency or grouping) must make at least one pin fail.  This is what shows
the pins are strong enough to trust the oracle."""
import inspect
import types

import pytest

import oracle.core as real
from oracle_pins import ALL_PINS

MUTANTS = {
    "rotation_sign": ("out[:, n_text:, :, c0 + 0:c0 + d_a:2] = xa * cos - xb * sin",
                      "out[:, n_text:, :, c0 + 0:c0 + d_a:2] = xa * cos + xb * sin"),
    "rotation_swap_sin_cos": ("xa * sin + xb * cos", "xa * cos + xb * sin"),
    "freq_whole_head": ("omega = theta ** (-2.0 * r / d_a)", "omega = theta ** (-2.0 * r / d)"),
    "freq_no_factor_2": ("omega = theta ** (-2.0 * r / d_a)", "omega = theta ** (-1.0 * r / d_a)"),
    "axis_order_swapped": ("phi = coords[:, axis]", "phi = coords[:, 2 - axis]"),
    "unfold_h_fastest": ("np.indices((t, h, w)).reshape(3, -1).T",
                         "np.indices((t, w, h)).reshape(3, -1).T[:, [0, 2, 1]]"),
    "half_split_pairs": ("xb = x[:, n_text:, :, c0 + 1:c0 + d_a:2]",
                         "xb = x[:, n_text:, :, c0 + 1 + (d_a // 2 - 1):c0 + d_a + (d_a // 2 - 1):2]"),
    "text_rotated": ("coords = video_coords(grid) + np.asarray(pos_offset, dtype=np.int64)[None, :]",
                     "coords = video_coords(grid) + np.asarray(pos_offset, dtype=np.int64)[None, :]\n"
                     "    x = np.concatenate([np.roll(x[:, :n_text], 1, axis=-1), x[:, n_text:]], axis=1)"),
    "grid_no_causal_plus1": ("t_lat = (frames - 1) // c_t + 1", "t_lat = frames // c_t"),
    "grid_no_patchify": ("return (t_lat // p_t, h_lat // p_s, w_lat // p_s)",
                         "return (t_lat, h_lat, w_lat)"),
    "single_skip_blocks": ("key = idx % k", "key = idx // (n // k)"),
    "group_size_wrong": ("key = (idx // k) % k", "key = (idx // (2 * k)) % k"),
    "group_as_single": ("key = (idx // k) % k", "key = idx % k"),
    "no_scale": ("s = sm_scale * (q @ k.T)", "s = (q @ k.T)"),
    "transposed_logits": ("s = sm_scale * (q @ k.T)", "s = sm_scale * (k @ q.T).T[:, ::-1]"),
    "no_normalise": ("o = (p @ v) / l", "o = (p @ v)"),
    "v_uses_q": ("o = (p @ v) / l", "o = (p @ q[:, :v.shape[1]] if q.shape[0] == v.shape[0] else p @ v) / l"),
    "lse_no_max": ("lse = (m + np.log(l))[:, 0]", "lse = (np.log(l))[:, 0]"),
    "default_scale_wrong": ("sm_scale = 1.0 / math.sqrt(d)", "sm_scale = 1.0 / d"),
    "k_not_rotated": ("k = rope3d(k, grid, n_text, rope_split, theta, pos_offset)", "pass"),
    "block_strided": ("key = idx // (n // k)", "key = idx % k"),
    "skiparse2d_axes_swapped": ("key = (hh % s) * s + (ww % s)", "key = (ww % s) * s + (hh % s)"),
    "skiparse2d_flat_index": ("key = (hh % s) * s + (ww % s)", "key = idx % k"),
    "skiparse2d_group_as_single": ("hh, ww = hh // s, ww // s", "hh, ww = hh, ww"),
    "skiparse2d_group_patch_s2": ("hh, ww = hh // s, ww // s", "hh, ww = hh // k, ww // k"),
    "block_runs_of_k": ("key = idx // (n // k)", "key = idx // k % k"),
    "bwd_no_row_term": ("ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))", "ds = p * dp"),
    "bwd_dk_from_ds_not_transposed": ("dk = sm_scale * (ds.T @ q)", "dk = sm_scale * (ds @ q)"),
    "bwd_dv_from_p_not_transposed": ("dv = p.T @ do", "dv = p @ do"),
    "bwd_dq_unscaled": ("dq = sm_scale * (ds @ k)", "dq = ds @ k"),
    "bwd_rope_forward_not_transpose": ("dq = rope3d_transpose(dq, grid, n_text, rope_split, theta, pos_offset)",
                                       "dq = rope3d(dq, grid, n_text, rope_split, theta, pos_offset)"),
    "rope_transpose_sign": ("out[:, n_text:, :, c0 + 0:c0 + d_a:2] = xa * cos + xb * sin",
                            "out[:, n_text:, :, c0 + 0:c0 + d_a:2] = xa * cos - xb * sin"),
    "perm_inverse_wrong": ("inv[perm] = np.arange(n, dtype=np.int64)", "inv[:] = perm"),
    "packed_global_positions": ("pos_offset=pos_offset, rope=rope,\n                          rows=out_rows[sel] - start)",
                                "pos_offset=(pos_offset[0] + start, pos_offset[1], pos_offset[2]), rope=rope,\n                          rows=out_rows[sel] - start)"),
    "packed_attends_across": ("        os_, ls_ = attn3d(q[:, start:end], k[:, start:end], v[:, start:end], grid=grid,",
                              "        os_, ls_ = attn3d(q[:, start:end], k[:, start:end], v[:, start:end] + v[:, :1].mean(), grid=grid,"),
    "packed_segment_off_by_one": ("        end = start + int(n_text) + int(np.prod(grid))",
                                  "        end = start + int(n_text) + int(np.prod(grid)) - (1 if start else 0)"),
}


def _mutant(name):
    old, new = MUTANTS[name]
    src = inspect.getsource(real)
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src.replace(old, new, 1), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _mutant(name)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # noqa: BLE001 -- any failure counts as caught
            failed.append((pin.__name__, type(e).__name__))
    assert failed, f"mutant {name} passed every pin"
