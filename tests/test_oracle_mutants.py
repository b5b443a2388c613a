"""The pins are strong enough: a plausible mistake planted anywhere in the
oracle must make at least one of them fail.

Each mutant is a copy of oracle/qr_oracle.c with one textual change, built
into a temporary library with the same flags (CPU only; nothing here touches
the HIP path).  Every replacement must match exactly once, so a later edit of
the oracle cannot silently turn a mutant into a no-op.
"""
import os

import pytest

import oracle
from oracle import build as obuild
import pins

SRC = open(obuild.SRC).read()

MUTANTS = {
    "scale_rounded_to_nearest": [
        ("double r = ceil(a / q) * q;", "double r = nearbyint(a / q) * q;")],
    "code_ties_away_from_zero": [
        ("float q = nearbyintf(t);", "float q = roundf(t);")],
    "code_bits_msb_first": [
        ("if ((code >> j) & 1u) blk[bit / 8] |= (uint8_t)(1u << (bit % 8));",
         "if ((code >> j) & 1u) blk[bit / 8] |= (uint8_t)(0x80u >> (bit % 8));")],
    "sum_in_reverse_rank_order": [
        ("for (int r = 0; r < W; r++) {\n      if (c == C_FP) {",
         "for (int r = W - 1; r >= 0; r--) {\n      if (c == C_FP) {"),
        ("acc[i] = (r == 0) ? v[i] : acc[i] + v[i];",
         "acc[i] = (r == W - 1) ? v[i] : acc[i] + v[i];")],
    "zero_rounded_to_nearest": [
        ("*z = ref_rd16(mn);", "*z = ref_f2h(mn);")],
    "no_constant_block_rule": [
        ("float arg = (mx == mn) ? a : a / qmax;", "float arg = a / qmax;")],
    "symmetric_range_off_by_one": [
        ("return (float)((1 << (b - 1)) - 1);", "return (float)(1 << (b - 1));")],
    "e4m3_subnormal_threshold": [
        ("if (a < ldexp(1.0, -6)) {\n    q = ldexp(1.0, -9);",
         "if (a < ldexp(1.0, -7)) {\n    q = ldexp(1.0, -9);")],
    "asym_dequant_drops_zero": [
        ("return p + ref_h2f(z);", "return p;")],
    "chunk_size_floor": [
        ("size_t bpc = (nb + (size_t)W - 1) / (size_t)W;",
         "size_t bpc = nb / (size_t)W;")],
    "f16_ties_up": [
        ("double r = nearbyint(a / q) * q;            /* a/q exact; nearbyint is RNE */",
         "double r = floor(a / q + 0.5) * q;")],
    "bf16_truncates": [
        ("double r = nearbyint(a / q) * q;\n  if (r >= ldexp(1.0, 128))",
         "double r = trunc(a / q) * q;\n  if (r >= ldexp(1.0, 128))")],
    "scale_plane_unaligned": [
        ("return align256(nblocks(n) * ref_block_code_bytes(c));",
         "return nblocks(n) * ref_block_code_bytes(c);")],
    "sign_extension_missing": [
        ("if (q & (1 << (b - 1))) q -= (1 << b);", "if (q & (1 << b)) q -= (1 << b);")],
    "absmax_from_max_only": [
        ("float a = fabsf(mx) > fabsf(mn) ? fabsf(mx) : fabsf(mn);", "float a = fabsf(mx);")],
    "asym_t_ignores_zero": [
        ("float t = (v[i] - fz) * inv;", "float t = v[i] * inv;")],
    "h2f_exponent_bias": [
        ("v = ldexp(1.0 + m / 1024.0, e - 15);", "v = ldexp(1.0 + m / 1024.0, e - 16);")],
    "e4m3_decode_subnormal_scale": [
        ("if (e == 0) v = ldexp((double)m, -9);", "if (e == 0) v = ldexp((double)m, -10);")],
    "rd16_negative_rounds_toward_zero": [
        ("if (a < 0.0) return 0x8000 | ref_ru16((float)-a);",
         "if (a < 0.0) return 0x8000 | ref_rd16((float)-a);")],
    "oneshot_sum_in_reverse_rank_order": [
        ("float acc = ld(dtype, xs[0][i]);\n    for (int r = 1; r < W; r++) acc = acc + ld(dtype, xs[r][i]);",
         "float acc = ld(dtype, xs[W - 1][i]);\n    for (int r = W - 2; r >= 0; r--) acc = acc + ld(dtype, xs[r][i]);")],
    "oneshot_rounds_every_add": [
        ("for (int r = 1; r < W; r++) acc = acc + ld(dtype, xs[r][i]);",
         "for (int r = 1; r < W; r++) acc = ld(dtype, st(dtype, acc + ld(dtype, xs[r][i])));")],
    "oneshot_range_in_elements": [
        ("size_t e_lo = blk_lo * BLK, e_hi = blk_hi * BLK < n ? blk_hi * BLK : n;",
         "size_t e_lo = blk_lo, e_hi = blk_hi < n ? blk_hi : n;")],
    "cast_input_not_rounded_to_fp16": [
        ("if (dtype == T_BF16_VIA_FP16) return ref_h2f(ref_f2h(ref_bf2f(x)));",
         "if (dtype == T_BF16_VIA_FP16) return ref_bf2f(x);")],
    "cast_output_skips_fp16": [
        ("if (dtype == T_BF16_VIA_FP16) return ref_f2bf(ref_h2f(ref_f2h(v)));",
         "if (dtype == T_BF16_VIA_FP16) return ref_f2bf(v);")],
    "cast_fp_wire_kept_bf16": [
        ("static int wire_type(int dtype) { return dtype == T_BF16_VIA_FP16 ? T_FP16 : dtype; }",
         "static int wire_type(int dtype) { return dtype == T_BF16_VIA_FP16 ? T_BF16 : dtype; }")],
    # stage 1 of the quantized codecs alone (the FP codec's sum kept as it is)
    "quantized_sum_in_reverse_rank_order": [
        ("for (int r = 0; r < W; r++) {\n      if (c == C_FP) {",
         "for (int rr = 0; rr < W; rr++) {\n      int r = (c == C_FP) ? rr : W - 1 - rr;\n"
         "      if (c == C_FP) {"),
        ("acc[i] = (r == 0) ? v[i] : acc[i] + v[i];",
         "acc[i] = (rr == 0) ? v[i] : acc[i] + v[i];")],
    "quantized_sum_in_binary64": [
        ("for (int i = 0; i < L; i++) acc[i] = (r == 0) ? v[i] : acc[i] + v[i];\n    }",
         "for (int i = 0; i < L; i++) {\n"
         "        if (c != C_FP) acc64[i] = (r == 0) ? (double)v[i] : acc64[i] + (double)v[i];\n"
         "        acc[i] = (r == 0) ? v[i] : acc[i] + v[i];\n"
         "      }\n    }\n"
         "    if (c != C_FP) for (int i = 0; i < L; i++) acc[i] = (float)acc64[i];"),
        ("float acc[BLK], v[BLK];\n    for (int r = 0; r < W; r++) {",
         "float acc[BLK], v[BLK];\n    double acc64[BLK];\n    for (int r = 0; r < W; r++) {")],
    "requantize_from_sums_rounded_to_buffer_type": [
        ("      wire_put_block(c, reduced, n, k, acc, L);",
         "      for (int i = 0; i < L; i++) acc[i] = ld(dtype, st(dtype, acc[i]));\n"
         "      wire_put_block(c, reduced, n, k, acc, L);")],
    "zero_plane_overlaps_scales": [
        ("return align256(ref_scale_offset(c, n) + 2 * nblocks(n));",
         "return align256(ref_scale_offset(c, n));")],
}


def _mutant_source(edits):
    src = SRC
    for old, new in edits:
        assert src.count(old) == 1, "mutation anchor not unique/present: %r" % old
        src = src.replace(old, new)
    return src


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    src = tmp_path / ("m_%s.c" % name)
    src.write_text(_mutant_source(MUTANTS[name]))
    lib = obuild.build(out=str(tmp_path / ("libm_%s.so" % name)), src=str(src))
    L = oracle.load_variant(lib)
    caught = []
    for check in pins.QUICK_CHECKS + [pins.check_h2f_exhaustive,
                                      pins.check_constants_exhaustive]:
        try:
            check(L)
        except AssertionError:
            caught.append(check.__name__)
            break
        except Exception as e:          # a crash in a check also counts
            caught.append("%s:%s" % (check.__name__, type(e).__name__))
            break
    assert caught, "planted mistake %r passed every pin" % name


def test_real_oracle_source_is_the_unmutated_one():
    for edits in MUTANTS.values():
        _mutant_source(edits)          # every anchor is present exactly once
    assert os.path.exists(obuild.SRC)
