/*
 * oracle.h -- declarations of the CPU oracle in oracle.c, for C and C++ test
 * programs.  TEST INFRASTRUCTURE ONLY: the product library never includes
 * this header or links the oracle.  Meanings, layouts and sources of every
 * argument are documented at the definitions in oracle.c.
 */
#ifndef ORACLE_H
#define ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_SHAPE (-2)
#define ORACLE_ERR_ROUTING (-3)

float oracle_bf16_to_float(uint16_t h);
uint16_t oracle_bf16_round(float f);
float oracle_e4m3_decode(uint8_t c);
uint8_t oracle_e4m3_encode(float q);
int oracle_layout(int P, int S, int E, int K, int A, int symmetric, const int64_t *topk_idx,
                  uint8_t *is_token_in_rank, int32_t *num_tokens_per_rank,
                  int32_t *num_tokens_per_expert, int32_t *rank_prefix_matrix,
                  int32_t *num_recv_tokens, int32_t *num_tokens_per_expert_total,
                  int64_t *expert_offset, int64_t *num_expanded, int64_t *window_row_base,
                  int32_t *dst_slot, int32_t *send_head, int32_t *recv_src_idx,
                  int64_t *recv_src_base);
void oracle_quantize_row(const uint16_t *x, int H, uint8_t *codes, float *scales);
void oracle_quantize_row_ue8m0(const uint16_t *x, int H, uint8_t *codes, uint8_t *exps);
void oracle_quantize_rows_ue8m0(const uint16_t *x, int H, int64_t row_begin, int64_t row_end,
                                uint8_t *codes, uint8_t *exps);
void oracle_quantize_rows(const uint16_t *x, int H, int64_t row_begin, int64_t row_end,
                          uint8_t *codes, float *scales);
int oracle_dispatch(int P, int S, int E, int K, int H, int A, int fp8, int zero_padding,
                    const int64_t *topk_idx, const int32_t *dst_slot,
                    const int32_t *num_tokens_per_expert_total, const int64_t *expert_offset,
                    const int64_t *window_row_base, const uint16_t *x, const float *topk_weights,
                    int64_t row_begin, int64_t row_end, void *recv_x, float *recv_scales,
                    float *recv_weights, int32_t *recv_src_meta);
int oracle_dispatch_general(int P, int S, int E, int K, int H, int A, int fp8, int zero_padding,
                            int scales_col_major, int64_t capacity, const int64_t *topk_idx,
                            const int32_t *dst_slot, const int32_t *num_tokens_per_expert_total,
                            const int64_t *expert_offset, const int64_t *window_row_base,
                            const uint16_t *x, const uint8_t *x_codes, const float *x_scales,
                            const float *topk_weights, int64_t row_begin, int64_t row_end,
                            void *recv_x, float *recv_scales, float *recv_weights,
                            int32_t *recv_src_meta, int64_t *dropped);
int oracle_combine(int P, int S, int E, int K, int H, const int64_t *topk_idx,
                   const int32_t *dst_slot, const int64_t *window_row_base, const uint16_t *y,
                   const float *topk_weights, int64_t tok_begin, int64_t tok_end, uint16_t *out);
int oracle_combine_general(int P, int S, int E, int K, int H, int64_t capacity,
                           const int64_t *topk_idx, const int32_t *dst_slot,
                           const int64_t *window_row_base, const uint16_t *y,
                           const float *topk_weights, const uint16_t *bias, int64_t tok_begin,
                           int64_t tok_end, uint16_t *out);

#ifdef __cplusplus
}
#endif

#endif /* ORACLE_H */
