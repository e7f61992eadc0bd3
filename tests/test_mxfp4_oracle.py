"""Pins of the oracle's MXFP4 expert-weight decoding (4-bit E2M1 elements in
blocks of 32 with an E8M0 power-of-two scale, OCP Microscaling Formats v1.0)
against the format's definition, torch's E8M0 decoding, brute force, and the
float32 layer on values every format holds exactly.

"Serving MoE models with expert parallelism on 8xH200", sections "Memory math
for 8xH200" (gpt-oss-120b in its native MXFP4) and "Quantization choices"
(4-bit expert weights halve the FP8 footprint again).
"""
import numpy as np
import torch

from oracle import moe_oracle as orc

# The E2M1 values the MX specification lists for codes 0..7 (sign = bit 3).
SPEC_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_table_matches_the_spec_list():
    tab = orc.e2m1_table()
    assert tab[:8].tolist() == SPEC_E2M1
    assert tab[8:].tolist() == [-v for v in SPEC_E2M1]
    assert np.signbit(tab[8])                     # code 8 is -0
    # every E2M1 value times any power of two in bf16's normal range is a bf16
    for k in (-120, -3, 0, 7, 120):
        v = tab * 2.0 ** k
        assert np.array_equal(torch.from_numpy(v).to(torch.bfloat16).double().numpy(), v)


def test_e8m0_matches_torch():
    s = np.arange(256)
    ours = orc.e8m0_to_f64(s)
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e8m0fnu)
    ref = ref.to(torch.float64).numpy()
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert np.array_equal(ours[:255], ref[:255])
    assert ours[127] == 1.0 and ours[0] == 2.0 ** -127 and ours[254] == 2.0 ** 127


def test_dequant_nibble_order_and_block_major_scales():
    # 3 rows, 96 columns (3 blocks of 32): scale s[b, r] distinct for every
    # (block, row), so a transposed scale index cannot pass; byte 0x72 holds
    # +1.0 (code 2) in its low nibble and +6.0 (code 7) in its high nibble
    R, C = 3, 96
    rng = np.random.default_rng(5)
    s = rng.permutation(np.arange(120, 120 + R * (C // 32))).reshape(C // 32, R).astype(np.uint8)
    q = np.full((R, C // 2), 0x72, dtype=np.uint8)
    got = orc.dequant_mxfp4(q, s)
    scale = np.repeat(np.exp2(s.T.astype(np.float64) - 127), 32, axis=1)   # [R, C]
    pattern = np.tile([1.0, 6.0], C // 2)
    assert np.array_equal(got, scale * pattern[None, :])


def test_dequant_random_codes_brute_force():
    R, C = 4, 64
    rng = np.random.default_rng(6)
    q = rng.integers(0, 256, size=(R, C // 2), dtype=np.uint8)
    s = rng.integers(100, 150, size=(C // 32, R), dtype=np.uint8)
    got = orc.dequant_mxfp4(q, s)
    for r in range(R):
        for c in range(C):
            byte = int(q[r, c // 2])
            code = (byte >> 4) if c % 2 else (byte & 0xF)
            mag = SPEC_E2M1[code & 7]
            want = (-mag if code & 8 else mag) * 2.0 ** (int(s[c // 32, r]) - 127)
            assert got[r, c] == want


def encode_mxfp4(w: np.ndarray, exps: np.ndarray):
    """Exact encoder for the test: w [R, C] whose block (r, b) values are
    E2M1 values times 2^exps[b, r]."""
    R, C = w.shape
    codes = np.zeros((R, C), dtype=np.uint8)
    for r in range(R):
        for c in range(C):
            v = w[r, c] / 2.0 ** int(exps[c // 32, r])
            mag = SPEC_E2M1.index(abs(v))
            codes[r, c] = mag | (8 if v < 0 else 0)
    q = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return q, (exps + 127).astype(np.uint8)


def test_mxfp4_path_equals_the_f32_path_on_shared_values():
    rng = np.random.default_rng(15)
    E_l, F, d, T, k = 2, 64, 96, 6, 1
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)

    def draw(E, R, C):
        exps = rng.integers(-3, 3, size=(E, C // 32, R))
        sign = rng.choice([-1.0, 1.0], size=(E, R, C))
        w = rng.choice(mags, size=(E, R, C)) * sign
        w = w * np.exp2(np.repeat(exps.transpose(0, 2, 1), 32, axis=2))
        return w.astype(np.float32), exps
    wg, eg = draw(E_l, F, d)
    wu, eu = draw(E_l, F, d)
    wd, ed = draw(E_l, d, F)
    x = rng.choice(mags, size=(T, d)).astype(np.float32)
    L = rng.standard_normal((T, E_l)).astype(np.float32)
    ref = orc.moe_layer_forward(x, L, k, wg, wu, wd, act_fmt="f32", weight_fmt="f32")["out"]
    enc = [list(zip(*[encode_mxfp4(w[j].astype(np.float64), e[j]) for j in range(E_l)]))
           for w, e in ((wg, eg), (wu, eu), (wd, ed))]
    (qg, sg), (qu, su), (qd, sd) = [(np.stack(a), np.stack(b)) for a, b in enc]
    xb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = orc.moe_layer_forward(xb, L, k, qg, qu, qd, act_fmt="bf16", weight_fmt="mxfp4",
                                s_gate=sg, s_up=su, s_down=sd)["out"]
    assert np.array_equal(got, ref)
