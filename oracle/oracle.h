/* oracle.h -- TEST INFRASTRUCTURE. Plain CPU definition of the MoE expert-parallel
 * dispatch/combine data path, used only to check the HIP implementation.
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may call it.
 * It shares no code, header or constant with the HIP library.
 *
 * All arrays are host memory, row-major, owned by the caller.
 * Return value: 0 on success, -1 on an argument the definition does not cover.
 */
#ifndef EP_ORACLE_H
#define EP_ORACLE_H
#include <stdint.h>

int oracle_layout(const int64_t *topk_idx, int64_t T, int k, int E, int R, int N,
                  int32_t *count_r, int32_t *count_n, int32_t *count_e,
                  uint8_t *in_rank, int32_t *rank_offset, int32_t *expert_offset,
                  int32_t *token_slot, int32_t *error_flag);

int oracle_dispatch(const uint16_t *x, const int64_t *topk_idx, const float *topk_w,
                    int64_t T, int H, int k, int E, int R, const int32_t *token_slot,
                    int64_t cap, uint16_t *recv_x, int64_t *recv_idx, float *recv_w,
                    int32_t *recv_src);

int oracle_restripe_prob(const uint32_t *prob, int64_t T, int N, int P, int64_t Tmax,
                         uint32_t *out);

int oracle_combine(const uint16_t *partial, int64_t rows, const int32_t *token_slot,
                   int64_t T, int H, int R, uint16_t *out);

int oracle_quantize_fp8(const uint16_t *x, int64_t T, int H, uint8_t *codes, float *scales);

int oracle_dispatch_fp8(const uint16_t *x, const int64_t *topk_idx, const float *topk_w,
                        int64_t T, int H, int k, int E, int R, const int32_t *token_slot,
                        int64_t cap, uint8_t *recv_codes, float *recv_scales,
                        int64_t *recv_idx, float *recv_w, int32_t *recv_src);

int oracle_node_slots(const int64_t *topk_idx, int64_t T, int k, int E, int R, int N,
                      int32_t *node_slot);

int oracle_restripe_prob_sparse(const uint32_t *prob, int64_t T, int N, int P,
                                const int32_t *node_slot, int64_t Tmax, uint32_t *out);

int oracle_expert_slots(const int64_t *topk_idx, int64_t T, int k, int E, int32_t *expert_slot);

int oracle_dispatch_permute(const uint16_t *x, const int64_t *topk_idx, const float *topk_w,
                            int64_t T, int H, int k, const int32_t *expert_slot, int64_t cap,
                            uint16_t *perm_x, float *perm_w, int32_t *perm_src);

int oracle_hook_dispatch_send(const uint16_t *x, const int64_t *topk_idx, const float *topk_w,
                              int64_t T, int H, int k, int N, const int32_t *node_slot,
                              int64_t Tmax, uint16_t *stage_x, int64_t *stage_idx,
                              float *stage_w, int32_t *stage_src);

int oracle_hook_dispatch_recv(const uint16_t *stage_x, const int64_t *stage_idx,
                              const float *stage_w, const int32_t *stage_src,
                              const int32_t *count_n, int N, int64_t Tmax, int H, int k, int E,
                              int R, const int32_t *token_slot, int64_t T, int64_t cap,
                              uint16_t *recv_x, int64_t *recv_idx, float *recv_w,
                              int32_t *recv_src);

int oracle_hook_combine_send(const uint16_t *partial, int64_t rows, const int32_t *token_slot,
                             int64_t T, int H, int R, int N, const int32_t *node_slot,
                             int64_t Tmax, uint16_t *stage);

int oracle_hook_combine_recv(const uint16_t *stage, int N, int64_t Tmax,
                             const int32_t *node_slot, int64_t T, int H, uint16_t *out);

uint8_t oracle_f32_to_e4m3(float v);
float oracle_e4m3_to_f32(uint8_t c);
void oracle_f32_to_e4m3_array(const float *in, int64_t n, uint8_t *out);

uint16_t oracle_f32_to_bf16(float f);
float oracle_bf16_to_f32(uint16_t b);
void oracle_f32_to_bf16_array(const float *in, int64_t n, uint16_t *out);

#endif
