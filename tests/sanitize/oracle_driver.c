/*
 * Host sanitizer driver for the C oracle (oracle/pqo.c): every entry point
 * on small arrays with the edge values the pins use (zeros, signed zeros,
 * bf16 max, subnormals, NaN-free random bits), built with
 * -fsanitize=address,undefined so an out-of-bounds access, overflow or
 * undefined shift fails the run.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void pqo_quantize_mxfp8_rowwise(const uint16_t *x, long R, long C, long ld, uint8_t *q, uint8_t *s);
void pqo_quantize_mxfp8_colwise(const uint16_t *x, long R, long C, long ld, uint8_t *qT, uint8_t *sT);
void pqo_quantize_nvfp4(const uint16_t *x, long R, long C, long ld, long rpg, uint8_t *q,
                        uint8_t *sb, float *sg);
void pqo_quantize_nvfp4_given_scale(const uint16_t *x, long R, long C, long ld, const float *sg,
                                    uint8_t *q, uint8_t *sb);
void pqo_quantize_fp8_block(const uint16_t *x, long R, long C, long ld, long br, uint8_t *q,
                            float *s);
void pqo_decode_fp8_block(const uint8_t *q, const float *s, long R, long C, long br, double *out);
void pqo_dequantize_mxfp8(const uint8_t *q, const uint8_t *s, long R, long C, uint16_t *y);
void pqo_dequantize_nvfp4(const uint8_t *q, const uint8_t *sb, const float *sg, long R, long C,
                          long rpg, uint16_t *y);
void pqo_decode_mxfp8(const uint8_t *q, const uint8_t *s, long R, long C, double *out);
void pqo_decode_nvfp4(const uint8_t *q, const uint8_t *sb, const float *sg, long R, long C,
                      long rpg, double *out);
long pqo_inexact_count(void);

static uint16_t edge(unsigned i, unsigned r)
{
    static const uint16_t e[] = {0x0000, 0x8000, 0x7F7F, 0xFF7F, 0x0001, 0x8001, 0x0080,
                                 0x3F80, 0xBF80, 0x4120, 0x43E0, 0x44E0, 0x3E80};
    if (i % 7 == 0)
        return e[(i / 7 + r) % (sizeof e / sizeof e[0])];
    uint16_t b = (uint16_t)((r * 2654435761u + i * 40503u) >> 7);
    if ((b & 0x7F80) == 0x7F80)
        b &= 0xBFFF; /* keep finite */
    return b;
}

int main(void)
{
    const long R = 256, C = 256; /* whole 128 x 128 blocks for block FP8 */
    uint16_t *x = malloc(R * C * 2);
    for (long i = 0; i < R * C; ++i)
        x[i] = edge((unsigned)i, (unsigned)(i / C));
    memset(x + 3 * C, 0, C * 2); /* a zero row */
    uint8_t *q = malloc(R * C), *s = malloc(R * C / 16), *qT = malloc(R * C), *sT = malloc(R * C / 32);
    float *sg = malloc(R * sizeof(float)), *fs = malloc((R * C / 128) * sizeof(float));
    uint16_t *y = malloc(R * C * 2);
    double *d = malloc(R * C * sizeof(double));
    pqo_quantize_mxfp8_rowwise(x, R, C, C, q, s);
    pqo_dequantize_mxfp8(q, s, R, C, y);
    pqo_decode_mxfp8(q, s, R, C, d);
    pqo_quantize_mxfp8_colwise(x, R, C, C, qT, sT);
    for (long rpg = 1; rpg <= R; rpg *= 16) {
        pqo_quantize_nvfp4(x, R, C, C, rpg, q, s, sg);
        pqo_dequantize_nvfp4(q, s, sg, R, C, rpg, y);
        pqo_decode_nvfp4(q, s, sg, R, C, rpg, d);
    }
    pqo_quantize_nvfp4(x, R, C, C, 1, q, s, sg);
    for (long r = 0; r < R; ++r)
        sg[r] = sg[r] * 4.0f; /* a larger running scale */
    pqo_quantize_nvfp4_given_scale(x, R, C, C, sg, q, s);
    for (long br = 1; br <= 128; br *= 128) {
        pqo_quantize_fp8_block(x, R, C, C, br, q, fs);
        pqo_decode_fp8_block(q, fs, R, C, br, d);
    }
    long inexact = pqo_inexact_count();
    printf("oracle driver done, inexact %ld\n", inexact);
    free(x); free(q); free(s); free(qT); free(sT); free(sg); free(fs); free(y); free(d);
    return inexact != 0;
}
