/* Seeded, counter-based synthetic inputs for the quantised MoE expert layer.
 *
 * This generator makes random inputs only; it holds none of the layer's arithmetic. The same
 * definitions are implemented twice, once here for the host and once in gen_fill.hip for the
 * GPU, and both must produce identical bytes for codes, scales and biases.
 *
 * Generator: SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014) used as a counter-based stream: draw(key, i) is the (i+1)-th output
 * of SplitMix64 seeded with `key`, i.e. mix64(key + (i+1)*0x9E3779B97F4A7C15).
 *
 * Streams are keyed by (seed, family, layer, tensor, expert, matrix); see bq_tensor_key.
 *  - codes:   element n of a matrix (row-major, n = r*cols + c) is field (n mod P) of draw(key, n div P),
 *             P = 64/bits fields of `bits` bits each, field 0 in the least significant bits.
 *  - uniform: element m is lo + (hi-lo)*t with t = (draw(key, m) >> 11) * 2^-53, evaluated in IEEE
 *             double with one rounding per operation (no fused multiply-add), then rounded to bf16
 *             with round-to-nearest-even.
 *  - ints:    element m is lo + (draw(key, m) mod (hi - lo + 1)), an integer in [lo, hi] (the
 *             E8M0 block scales of MXFP4 experts).
 *  - normal:  element m is sigma*sqrt(-2 ln u1)*cos(2 pi u2) (Box and Muller, 1958) with
 *             u1 = ((draw(key,2m) >> 11) + 1) * 2^-53 and u2 = (draw(key,2m+1) >> 11) * 2^-53; host only.
 */
#ifndef BQ_SYNTH_GEN_H
#define BQ_SYNTH_GEN_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum bq_tensor_id {
  BQ_T_X = 1,           /* token activations, fp32 [T][H] */
  BQ_T_ROUTER = 2,      /* router weights, bf16 [E][H] */
  BQ_T_SHARED_GATE = 3, /* shared-expert gate vector, bf16 [H] */
  BQ_T_CODES = 4,       /* expert matrix codes, one byte per element */
  BQ_T_SCALE = 5,       /* expert matrix scales, bf16 per (row, group) */
  BQ_T_BIAS = 6         /* expert matrix biases, bf16 per (row, group) */
};

uint64_t bq_mix64(uint64_t z);
uint64_t bq_draw(uint64_t key, uint64_t i);
uint64_t bq_tensor_key(uint64_t seed, int64_t family, int64_t layer, int64_t tensor, int64_t expert,
                       int64_t matrix);
uint16_t bq_bf16_rne(double v);

/* codes: elements [start, start+n) of the stream, one byte each (0..2^bits-1). bits is 2 or 4. */
void bq_gen_codes(uint64_t key, int bits, int64_t start, int64_t n, uint8_t* out);
/* uniform bf16 in [lo, hi] (before rounding): elements [start, start+n). */
void bq_gen_uniform_bf16(uint64_t key, double lo, double hi, int64_t start, int64_t n, uint16_t* out);
/* integers in [lo, hi] (0 <= lo <= hi <= 65535), one uint16 each: elements [start, start+n). */
void bq_gen_ints_u16(uint64_t key, int lo, int hi, int64_t start, int64_t n, uint16_t* out);
/* normal(0, sigma) rounded to bf16 / to fp32 / left in fp64: elements [start, start+n). */
void bq_gen_normal_bf16(uint64_t key, double sigma, int64_t start, int64_t n, uint16_t* out);
void bq_gen_normal_f32(uint64_t key, double sigma, int64_t start, int64_t n, float* out);

#ifdef __cplusplus
}
#endif
#endif
