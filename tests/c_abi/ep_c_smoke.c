/* ep_c_smoke.c -- a plain C consumer of the C ABI in include/ep.h (no Python, no torch):
 * device buffers from the HIP runtime, one batch through the path on one stream in three
 * forms -- ep_get_layout, ep_dispatch, ep_restripe_prob, ep_combine; then the counts path,
 * ep_layout_counts (with the restripe), ep_dispatch_layout, ep_combine; then
 * ep_layout_dispatch (layout, dispatch and restripe in one launch), ep_combine -- each
 * time with the outputs pre-filled with a sentinel, copied back and compared bit for bit
 * with the CPU
 * oracle (TEST INFRASTRUCTURE, linked only into this test program).
 *
 * Inputs: T = 256 tokens, hidden 1024, 16 experts, top-4 distinct experts per token,
 * 4 ranks, 2 nodes, 8 prob floats per (token, node); values from a fixed xorshift stream.
 * Exit status 0 when every output matches, 1 on a mismatch, 2 on an API error. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "ep.h"
#include "oracle.h"

enum { T = 256, H = 1024, E = 16, K = 4, R = 4, N = 2, P = 8, TMAX = 256 };

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) {
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return rng_state;
}

#define HIP_OK(call)                                                        \
    do {                                                                    \
        hipError_t e_ = (call);                                             \
        if (e_ != hipSuccess) {                                             \
            fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));      \
            return 2;                                                       \
        }                                                                   \
    } while (0)
#define EP_OK_(call)                                                        \
    do {                                                                    \
        int s_ = (call);                                                    \
        if (s_ != EP_OK) {                                                  \
            fprintf(stderr, "%s: %s\n", #call, ep_status_string(s_));       \
            return 2;                                                       \
        }                                                                   \
    } while (0)

static int same(const char *what, const void *a, const void *b, size_t bytes) {
    if (memcmp(a, b, bytes) == 0) return 1;
    fprintf(stderr, "mismatch in %s\n", what);
    return 0;
}

int main(void) {
    const int64_t cap = (int64_t)T * (K < R ? K : R);
    /* host inputs: distinct experts per token, bf16 rows with small exponents, prob words */
    static int64_t idx[T * K];
    static float w[T * K];
    static uint16_t x[T * H], partial[T * K * H];
    static uint32_t prob[T * N * P];
    for (int t = 0; t < T; ++t) {
        int used[E] = {0};
        for (int j = 0; j < K; ++j) {
            int e;
            do e = (int)(next_u64() % E); while (used[e]);
            used[e] = 1;
            idx[t * K + j] = e;
            w[t * K + j] = (float)(next_u64() % 1000) / 1000.0f;
        }
    }
    for (int i = 0; i < T * H; ++i) x[i] = (uint16_t)(0x3C00 + (next_u64() % 0x0600)) ^ ((next_u64() & 1) << 15);
    for (int64_t i = 0; i < cap * H; ++i) partial[i] = (uint16_t)(0x3C00 + (next_u64() % 0x0600)) ^ ((next_u64() & 1) << 15);
    for (int i = 0; i < T * N * P; ++i) prob[i] = (uint32_t)next_u64();

    /* device buffers */
    hipStream_t st;
    HIP_OK(hipStreamCreate(&st));
    int64_t *d_idx; float *d_w; uint16_t *d_x, *d_partial, *d_recv_x, *d_out; uint32_t *d_prob, *d_prob_out;
    int32_t *d_cr, *d_cn, *d_ce, *d_ro, *d_eo, *d_slot, *d_src, *d_err; uint8_t *d_in; void *d_ws;
    int64_t *d_ridx; float *d_rw;
    const size_t ws_bytes = ep_layout_workspace_bytes(T, E, R, N);
    HIP_OK(hipMalloc((void **)&d_idx, sizeof idx));
    HIP_OK(hipMalloc((void **)&d_w, sizeof w));
    HIP_OK(hipMalloc((void **)&d_x, sizeof x));
    HIP_OK(hipMalloc((void **)&d_partial, sizeof partial));
    HIP_OK(hipMalloc((void **)&d_prob, sizeof prob));
    HIP_OK(hipMalloc((void **)&d_prob_out, sizeof(uint32_t) * N * TMAX * P));
    HIP_OK(hipMalloc((void **)&d_cr, sizeof(int32_t) * R));
    HIP_OK(hipMalloc((void **)&d_cn, sizeof(int32_t) * N));
    HIP_OK(hipMalloc((void **)&d_ce, sizeof(int32_t) * E));
    HIP_OK(hipMalloc((void **)&d_ro, sizeof(int32_t) * (R + 1)));
    HIP_OK(hipMalloc((void **)&d_eo, sizeof(int32_t) * (E + 1)));
    HIP_OK(hipMalloc((void **)&d_slot, sizeof(int32_t) * T * R));
    HIP_OK(hipMalloc((void **)&d_in, (size_t)T * R));
    HIP_OK(hipMalloc((void **)&d_err, sizeof(int32_t)));
    HIP_OK(hipMalloc(&d_ws, ws_bytes));
    HIP_OK(hipMalloc((void **)&d_recv_x, sizeof(uint16_t) * cap * H));
    HIP_OK(hipMalloc((void **)&d_ridx, sizeof(int64_t) * cap * K));
    HIP_OK(hipMalloc((void **)&d_rw, sizeof(float) * cap * K));
    HIP_OK(hipMalloc((void **)&d_src, sizeof(int32_t) * cap));
    HIP_OK(hipMalloc((void **)&d_out, sizeof(uint16_t) * T * H));
    HIP_OK(hipMemcpy(d_idx, idx, sizeof idx, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_w, w, sizeof w, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_x, x, sizeof x, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_partial, partial, sizeof partial, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_prob, prob, sizeof prob, hipMemcpyHostToDevice));

    void *d_cws;  /* the counts path's workspace: zero-filled once before its first use */
    const size_t cws_bytes = ep_layout_counts_workspace_bytes(T, E, R, N);
    HIP_OK(hipMalloc(&d_cws, cws_bytes));
    HIP_OK(hipMemset(d_cws, 0, cws_bytes));

    /* the oracle on the same inputs */
    static int32_t o_cr[R], o_cn[N], o_ce[E], o_ro[R + 1], o_eo[E + 1], o_slot[T * R], o_src[T * K], o_err;
    static uint8_t o_in[T * R];
    static uint16_t o_recv_x[T * K * H], o_out[T * H];
    static int64_t o_ridx[T * K * K];
    static float o_rw[T * K * K];
    static uint32_t o_prob[N * TMAX * P];
    if (oracle_layout(idx, T, K, E, R, N, o_cr, o_cn, o_ce, o_in, o_ro, o_eo, o_slot, &o_err) != 0 ||
        oracle_dispatch(x, idx, w, T, H, K, E, R, o_slot, cap, o_recv_x, o_ridx, o_rw, o_src) != 0 ||
        oracle_restripe_prob(prob, T, N, P, TMAX, o_prob) != 0 ||
        oracle_combine(partial, cap, o_slot, T, H, R, o_out) != 0) {
        fprintf(stderr, "oracle rejected the inputs\n");
        return 2;
    }
    const int64_t M = o_ro[R];

    static int32_t cr[R], cn[N], ce[E], ro[R + 1], eo[E + 1], slot[T * R], src[T * K], err;
    static uint8_t in_rank[T * R];
    static uint16_t recv_x[T * K * H], out[T * H];
    static int64_t ridx[T * K * K];
    static float rw[T * K * K];
    static uint32_t prob_out[N * TMAX * P];
    int ok = 1;
    for (int form = 0; form < 3; ++form) {
        /* outputs pre-filled with a sentinel, so an element left unwritten shows */
        HIP_OK(hipMemset(d_cr, 0xAB, sizeof(int32_t) * R));
        HIP_OK(hipMemset(d_cn, 0xAB, sizeof(int32_t) * N));
        HIP_OK(hipMemset(d_ce, 0xAB, sizeof(int32_t) * E));
        HIP_OK(hipMemset(d_ro, 0xAB, sizeof(int32_t) * (R + 1)));
        HIP_OK(hipMemset(d_eo, 0xAB, sizeof(int32_t) * (E + 1)));
        HIP_OK(hipMemset(d_slot, 0xAB, sizeof(int32_t) * T * R));
        HIP_OK(hipMemset(d_in, 0xAB, (size_t)T * R));
        HIP_OK(hipMemset(d_err, 0xAB, sizeof(int32_t)));
        HIP_OK(hipMemset(d_recv_x, 0xAB, sizeof(uint16_t) * cap * H));
        HIP_OK(hipMemset(d_ridx, 0xAB, sizeof(int64_t) * cap * K));
        HIP_OK(hipMemset(d_rw, 0xAB, sizeof(float) * cap * K));
        HIP_OK(hipMemset(d_src, 0xAB, sizeof(int32_t) * cap));
        HIP_OK(hipMemset(d_prob_out, 0xAB, sizeof(uint32_t) * N * TMAX * P));
        HIP_OK(hipMemset(d_out, 0xAB, sizeof(uint16_t) * T * H));
        HIP_OK(hipDeviceSynchronize());

        /* the path, stream-ordered */
        if (form == 0) {
            EP_OK_(ep_get_layout(d_idx, T, K, E, R, N, d_cr, d_cn, d_ce, d_in, d_ro, d_eo, d_slot, NULL,
                                 NULL, d_err, d_ws, ws_bytes, st));
            EP_OK_(ep_dispatch(d_x, d_idx, d_w, T, H, K, E, R, d_slot, d_recv_x, d_ridx, d_rw, d_src,
                               cap, d_err, st));
            EP_OK_(ep_restripe_prob((const float *)d_prob, T, N, P, TMAX, (float *)d_prob_out, st));
        } else if (form == 1) {
            EP_OK_(ep_layout_counts(d_idx, T, K, E, R, N, d_err, NULL, (const float *)d_prob, P,
                                    TMAX, (float *)d_prob_out, d_cws, cws_bytes, st));
            EP_OK_(ep_dispatch_layout(d_x, d_idx, d_w, T, H, K, E, R, N, d_cr, d_ro, d_cn, d_ce, d_eo,
                                      d_slot, d_in, d_recv_x, d_ridx, d_rw, d_src, cap, d_err,
                                      d_cws, cws_bytes, st));
        } else {
            EP_OK_(ep_layout_dispatch(d_x, d_idx, d_w, T, H, K, E, R, N, d_cr, d_ro, d_cn, d_ce, d_eo,
                                      d_slot, d_in, d_recv_x, d_ridx, d_rw, d_src, cap,
                                      (const float *)d_prob, P, TMAX, (float *)d_prob_out, d_err,
                                      st));
        }
        EP_OK_(ep_combine(d_partial, cap, d_slot, T, H, R, d_out, d_err, st));
        HIP_OK(hipStreamSynchronize(st));

        /* results */
        HIP_OK(hipMemcpy(cr, d_cr, sizeof cr, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(cn, d_cn, sizeof cn, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(ce, d_ce, sizeof ce, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(ro, d_ro, sizeof ro, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(eo, d_eo, sizeof eo, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(slot, d_slot, sizeof slot, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(in_rank, d_in, sizeof in_rank, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(&err, d_err, sizeof err, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(recv_x, d_recv_x, sizeof(uint16_t) * cap * H, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(ridx, d_ridx, sizeof(int64_t) * cap * K, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(rw, d_rw, sizeof(float) * cap * K, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(src, d_src, sizeof(int32_t) * cap, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(prob_out, d_prob_out, sizeof prob_out, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(out, d_out, sizeof out, hipMemcpyDeviceToHost));

        const char *name = form == 0 ? "four calls" : form == 1 ? "counts path" : "one launch";
        int f_ok = 1;
        f_ok &= err == 0 && o_err == 0;
        f_ok &= same("num_tokens_per_rank", cr, o_cr, sizeof cr);
        f_ok &= same("num_tokens_per_node", cn, o_cn, sizeof cn);
        f_ok &= same("num_tokens_per_expert", ce, o_ce, sizeof ce);
        f_ok &= same("rank_offset", ro, o_ro, sizeof ro);
        f_ok &= same("expert_offset", eo, o_eo, sizeof eo);
        f_ok &= same("token_slot", slot, o_slot, sizeof slot);
        f_ok &= same("is_token_in_rank", in_rank, o_in, sizeof in_rank);
        f_ok &= same("recv_x", recv_x, o_recv_x, sizeof(uint16_t) * M * H);
        f_ok &= same("recv_topk_idx", ridx, o_ridx, sizeof(int64_t) * M * K);
        f_ok &= same("recv_topk_weights", rw, o_rw, sizeof(float) * M * K);
        f_ok &= same("recv_src_idx", src, o_src, sizeof(int32_t) * M);
        f_ok &= same("prob_dest_major", prob_out, o_prob, sizeof prob_out);
        f_ok &= same("combine out", out, o_out, sizeof out);
        /* receive rows past M keep the sentinel */
        for (int64_t i = M * H; i < cap * H; ++i)
            if (recv_x[i] != 0xABAB) {
                fprintf(stderr, "recv_x written past row M\n");
                f_ok = 0;
                break;
            }
        printf("ep_c_smoke: %s %s\n", name, f_ok ? "ok" : "MISMATCH");
        ok &= f_ok;
    }
    printf("ep_c_smoke: T=%d M=%lld %s\n", T, (long long)M, ok ? "ok" : "MISMATCH");
    return ok ? 0 : 1;
}
