"""Plant one plausible mistake at a time in a copy of the oracle (on the CPU)
and check that the oracle's pins (tests/test_oracle.py) reject it.

This is evidence that the pins constrain every part of the oracle: a
mistake that survived would mean some part of it is unpinned.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (original text in oracle/attention.py, planted mistake)
MUTATIONS = [
    ("s = scale * (q[r0:r1] @ k.T)", "s = (q[r0:r1] @ k.T)"),                     # dropped scale
    ("lse2[idx] = (m[:, 0] + np.log(l[:, 0])) / _LN2",
     "lse2[idx] = (m[:, 0] + np.log(l[:, 0]))"),                                   # natural-log LSE
    ("+ (lk - lq) + 1, 0, lk)", "+ 1, 0, lk)"),                                    # top-left causal
    ("+ (lk - lq) + 1, 0, lk)", "+ (lk - lq), 0, lk)"),                            # diagonal excluded
    ("by_req_head.setdefault((b, h // group), []).append(n)\n    for (b, g), members in by_req_head.items():\n        lk = int(seq_lens[b])",
     "by_req_head.setdefault((b, h % hkv), []).append(n)\n    for (b, g), members in by_req_head.items():\n        lk = int(seq_lens[b])"),  # interleaved GQA map
    ("physical = int(block_table_row[logical])", "physical = logical"),           # logical as physical page
    ("o[idx] = (e @ v) / l", "o[idx] = (e @ v)"),                                  # missing normalisation
    ("e = np.exp(s - m)", "e = np.exp(m - s)"),                                    # flipped sign
    ("np.exp2(exp.astype(np.float64) - 7.0)", "np.exp2(exp.astype(np.float64) - 8.0)"),  # FNUZ-style bias
    ("subnormal = man * 2.0 ** -9", "subnormal = man * 2.0 ** -10"),              # wrong subnormal step
    ("np.exp2(lse_parts - top_safe[None, :])", "np.exp(lse_parts - top_safe[None, :])"),  # merge in wrong base
    ("alpha = np.where(np.isfinite(m), np.exp(m - m_new), 0.0)",
     "alpha = np.where(np.isfinite(m), 1.0, 0.0)"),                                # recurrence without rescale
    ("return np.maximum(0, i + (lk - lq - window_left))",
     "return np.maximum(0, i + (lk - lq - window_left) + 1)"),                   # window one key short
    ("visible = (cols[None, :] < key_bound[r0:r1, None]) & (cols[None, :] >= key_start[r0:r1, None])",
     "visible = (cols[None, :] < key_bound[r0:r1, None]) & (cols[None, :] > key_start[r0:r1, None])"),  # start excluded
    ("widen_e4m3fn(v_codes, v_scale), cu_seqlens_q", "widen_e4m3fn(v_codes, k_scale), cu_seqlens_q"),  # FP8 V scale
    ("return prefill_dense(widen_e4m3fn(q_codes, q_scale), widen_e4m3fn(k_codes, k_scale),",
     "return prefill_dense(widen_e4m3fn(q_codes, 1.0), widen_e4m3fn(k_codes, k_scale),"),  # FP8 q scale dropped
    ("for n in members]), q_format, q_scale)", "for n in members]), q_format)"),   # decode q scale dropped
    ("rows.append(cache[physical, :take, head, :width])",
     "rows.append(cache[physical, :page_size, head, :width][:take])"),             # harmless: must survive
]


# (original text in oracle/cache.py, planted mistake), caught by tests/test_oracle_cache.py
CACHE_MUTATIONS = [
    ("take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))", "take_hi = (d_hi <= d_lo)"),   # ties away
    ("return np.where(np.isnan(y), np.uint8(0x7F), out)",
     "return np.where(np.isnan(y) | (np.abs(y) > E4M3_MAX), np.uint8(0x7F), out)"),            # overflow to NaN
    ("y = np.asarray(x, dtype=np.float32) / np.float32(scale)",
     "y = np.asarray(x, dtype=np.float64) / float(scale)"),                                    # exact quotient
    ("y = np.asarray(x, dtype=np.float32) / np.float32(scale)",
     "y = np.asarray(x, dtype=np.float32) * np.float32(scale)"),                               # scale multiplies
    ("(1.0 + m / 8.0) * 2.0 ** (e - 7)", "(1.0 + m / 8.0) * 2.0 ** (e - 8)"),                  # FNUZ bias
    ("row = int(layer_base_rows) + max(int(slot), 0)", "row = max(int(layer_base_rows) + int(slot), 0)"),  # clamp after base
    ("k = np.concatenate([widen_bf16(k_nope), rope], axis=-1)",
     "k = np.concatenate([rope, widen_bf16(k_nope)], axis=-1)"),                               # rope first
]


def _run_pins(tmp_root, test_file="test_oracle.py"):
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                           os.path.join("tests", test_file)],
                          cwd=tmp_root, env=env, capture_output=True, text=True, timeout=600)


@pytest.mark.parametrize("idx", range(len(MUTATIONS)))
def test_planted_mistake_is_caught(idx, tmp_path):
    original, planted = MUTATIONS[idx]
    shutil.copytree(os.path.join(ROOT, "oracle"), tmp_path / "oracle")
    (tmp_path / "tests").mkdir()
    for name in ("conftest.py", "test_oracle.py"):
        shutil.copy(os.path.join(ROOT, "tests", name), tmp_path / "tests" / name)
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), tmp_path / "tests" / "golden")
    src_path = tmp_path / "oracle" / "attention.py"
    src = src_path.read_text()
    assert original in src, "mutation anchor not found; update the list"
    src_path.write_text(src.replace(original, planted, 1))
    result = _run_pins(tmp_path)
    harmless = idx == len(MUTATIONS) - 1
    if harmless:
        assert result.returncode == 0, result.stdout[-2000:]
    else:
        assert result.returncode != 0, f"planted mistake survived the pins: {planted!r}"


@pytest.mark.parametrize("idx", range(len(CACHE_MUTATIONS)))
def test_planted_cache_mistake_is_caught(idx, tmp_path):
    original, planted = CACHE_MUTATIONS[idx]
    shutil.copytree(os.path.join(ROOT, "oracle"), tmp_path / "oracle")
    (tmp_path / "tests").mkdir()
    for name in ("conftest.py", "test_oracle_cache.py"):
        shutil.copy(os.path.join(ROOT, "tests", name), tmp_path / "tests" / name)
    src_path = tmp_path / "oracle" / "cache.py"
    src = src_path.read_text()
    assert original in src, "mutation anchor not found; update the list"
    src_path.write_text(src.replace(original, planted, 1))
    result = _run_pins(tmp_path, "test_oracle_cache.py")
    assert result.returncode != 0, f"planted mistake survived the pins: {planted!r}"
