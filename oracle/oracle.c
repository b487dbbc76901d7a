/* oracle.c -- TEST INFRASTRUCTURE, not part of the product path.
 *
 * A plain, slow, single-threaded CPU definition of the four steps of the
 * single-GPU core of MoE expert-parallel (EP) dispatch/combine:
 *   layout   : per-rank / per-node / per-expert token counts, the token-in-rank
 *              bitmap, exclusive prefix offsets and each (token, rank) receive slot;
 *   dispatch : copy each token's bf16 row and its rank-local top-k view, in
 *              ascending token order, into destination-major receive rows;
 *   restripe : prob [T][N][P] -> [N][Tmax][P];
 *   combine  : per token, sum its per-rank partial rows in fp32, round to bf16.
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * call it. It shares no code with the HIP library and uses nothing but libc.
 *
 * Sources (DeepEP pull-request pages):
 *  - "[PR #347] Feature/sm free normal kernel": names get_dispatch_layout
 *    (commit list) and fixes the workload (section 3.1).
 *  - "[PR #634] Hybrid ep nixl restripe": sections "Baseline problem" and
 *    "Fix" define the prob layouts and the restripe; its commit list names
 *    the scan/permute fusion with a per-local-expert sum array.
 *  - "[PR #453] ... Zero-Copy and TMA Offloading": a guard against too many
 *    received tokens (commit list), here a capacity check.
 * Where the pages leave a step open the plainest reading is taken:
 *  - expert e lives on rank e / (E/R); rank r on node r / (R/N);
 *  - a token counts once per rank, however many of its experts the rank holds;
 *  - per-expert counts count every (token, slot) pair;
 *  - expert id -1 is a masked slot (skipped); ids < -1 or >= E are skipped and
 *    raise the error flag;
 *  - a rank's receive rows are its tokens in ascending token order, ranks packed
 *    one after another at the exclusive prefix of the per-rank counts;
 *  - a receive row's top-k view keeps all k slots in order: the rank-local
 *    expert id (e - r*E/R) and its weight where the expert is on that rank,
 *    else -1 and +0.0f;
 *  - combine is an unweighted sum in ascending rank order, fp32, from +0.0f,
 *    then one round-to-nearest-even to bf16;
 *  - FP8 dispatch ("[PR #347]" section 3.2.1 and "[PR #453]" measure dispatch with an
 *    FP8 payload; their byte counts fit one fp32 scale per 128 channels): each token
 *    is quantised once, per group of 128 channels, to OCP e4m3 (4 exponent bits,
 *    bias 7, 3 mantissa bits, largest finite 448, no infinities): amax = largest
 *    |x| in the group, scale = amax / 448, code = e4m3(x * (448 / amax)) rounded to
 *    nearest even with the magnitude saturated at 448; an all-zero group gets scale 1
 *    and zero codes. Every destination row receives the same codes and scales;
 *  - dispatch + permute ("[PR #634]" measures "dispatch+permute"; its commit list
 *    names the scan over tokens per local expert): every valid (token, slot) pair
 *    gets its own row, rows grouped by expert id (so each rank's local experts are one
 *    contiguous range) and ordered by (token, slot) within an expert; a row carries
 *    the token's hidden row, the slot's weight and the source token;
 *  - sparse restripe ("[PR #634]", section "Fix": one put per run in the sparse
 *    path): only the (token, node) slices of tokens with a destination on the node are
 *    moved, packed at the start of the node's block in token order, so the slices of
 *    any run of consecutive tokens routed to a node are contiguous.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* bf16 is the top half of an IEEE-754 binary32 word. */
float oracle_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round a binary32 value to the nearest bf16, ties to even; a NaN stays a
 * (quiet) NaN. Adding 0x7fff plus the lowest kept bit carries into the kept
 * half exactly when the dropped half is above one half ulp, or equal to it
 * with an odd kept half. */
uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t kept_lsb = (u >> 16) & 1u;
    u += 0x7fffu + kept_lsb;
    return (uint16_t)(u >> 16);
}

void oracle_f32_to_bf16_array(const float *in, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f32_to_bf16(in[i]);
}

/* OCP e4m3 code of a finite fp32 value: round to nearest even on the e4m3 grid
 * (spacing 2^(e-3) in binade [2^e, 2^(e+1)) for e >= -6, 2^-9 below 2^-6), with the
 * magnitude saturated at 448. A NaN gives the NaN code 0x7f with the input's sign. */
uint8_t oracle_f32_to_e4m3(float v)
{
    const uint8_t sign = signbit(v) ? 0x80 : 0x00;
    if (isnan(v))
        return sign | 0x7f;
    const float a = fabsf(v);
    if (a >= 464.0f) /* at or beyond the midpoint between 448 and the next step */
        return sign | 0x7e;
    if (a == 0.0f)
        return sign;
    int e2;
    frexpf(a, &e2);        /* a = m * 2^e2, m in [0.5, 1) */
    int ex = e2 - 1;       /* a in [2^ex, 2^(ex+1)) */
    if (ex < -6)
        ex = -6;           /* subnormal range: quantum 2^-9 */
    float q = rintf(ldexpf(a, 3 - ex)); /* a in units of the quantum, nearest even */
    if (q >= 16.0f) {      /* rounded up into the next binade */
        ex += 1;
        q = 8.0f;
    }
    if (q < 8.0f)          /* subnormal */
        return sign | (uint8_t)q;
    return sign | (uint8_t)(((ex + 7) << 3) | ((int)q - 8));
}

float oracle_e4m3_to_f32(uint8_t c)
{
    const int s = c >> 7, ef = (c >> 3) & 0xf, m = c & 7;
    float v;
    if (ef == 0xf && m == 7)
        v = NAN;
    else if (ef == 0)
        v = ldexpf((float)m, -9);
    else
        v = ldexpf((float)(8 + m), ef - 7 - 3);
    return s ? -v : v;
}

void oracle_f32_to_e4m3_array(const float *in, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f32_to_e4m3(in[i]);
}

/* Per token and per group of 128 channels: scale = amax / 448, codes of x * (448/amax). */
int oracle_quantize_fp8(const uint16_t *x, int64_t T, int H, uint8_t *codes, float *scales)
{
    if (T < 0 || H < 128 || H % 128 != 0)
        return -1;
    const int G = H / 128;
    for (int64_t t = 0; t < T; ++t)
        for (int g = 0; g < G; ++g) {
            const uint16_t *xg = x + t * H + g * 128;
            float amax = 0.0f;
            for (int c = 0; c < 128; ++c) {
                const float a = fabsf(oracle_bf16_to_f32(xg[c]));
                if (a > amax)
                    amax = a;
            }
            const float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
            const float inv = amax > 0.0f ? 448.0f / amax : 1.0f;
            scales[t * G + g] = scale;
            for (int c = 0; c < 128; ++c)
                codes[t * H + g * 128 + c] = oracle_f32_to_e4m3(oracle_bf16_to_f32(xg[c]) * inv);
        }
    return 0;
}

/* Layout ("get_dispatch_layout", PR #347 commit list; scan over tokens per
 * local expert, PR #634 commit list). */
int oracle_layout(const int64_t *topk_idx, int64_t T, int k, int E, int R, int N,
                  int32_t *count_r, int32_t *count_n, int32_t *count_e,
                  uint8_t *in_rank, int32_t *rank_offset, int32_t *expert_offset,
                  int32_t *token_slot, int32_t *error_flag)
{
    if (T < 0 || k < 1 || E < 1 || R < 1 || N < 1 || E % R != 0 || R % N != 0 || k > E)
        return -1;
    const int experts_per_rank = E / R;
    const int ranks_per_node = R / N;
    int32_t flag = 0;

    for (int r = 0; r < R; ++r) count_r[r] = 0;
    for (int n = 0; n < N; ++n) count_n[n] = 0;
    for (int e = 0; e < E; ++e) count_e[e] = 0;

    for (int64_t t = 0; t < T; ++t) {
        uint8_t *row = in_rank + t * R;
        for (int r = 0; r < R; ++r) row[r] = 0;
        for (int j = 0; j < k; ++j) {
            int64_t e = topk_idx[t * k + j];
            if (e == -1)
                continue;
            if (e < -1 || e >= E) {
                flag = 1;
                continue;
            }
            count_e[e] += 1;
            row[e / experts_per_rank] = 1;
        }
        for (int r = 0; r < R; ++r)
            if (row[r])
                count_r[r] += 1;
        for (int n = 0; n < N; ++n) {
            int any = 0;
            for (int q = 0; q < ranks_per_node; ++q)
                if (row[n * ranks_per_node + q])
                    any = 1;
            if (any)
                count_n[n] += 1;
        }
    }

    rank_offset[0] = 0;
    for (int r = 0; r < R; ++r)
        rank_offset[r + 1] = rank_offset[r] + count_r[r];
    if (expert_offset) {
        expert_offset[0] = 0;
        for (int e = 0; e < E; ++e)
            expert_offset[e + 1] = expert_offset[e] + count_e[e];
    }

    /* Slot of (t, r): the rank's base row plus the number of earlier tokens
     * that also go to r. */
    int32_t *filled = (int32_t *)calloc((size_t)R, sizeof(int32_t));
    if (!filled)
        return -1;
    for (int64_t t = 0; t < T; ++t)
        for (int r = 0; r < R; ++r) {
            if (in_rank[t * R + r]) {
                token_slot[t * R + r] = rank_offset[r] + filled[r];
                filled[r] += 1;
            } else {
                token_slot[t * R + r] = -1;
            }
        }
    free(filled);
    *error_flag = flag;
    return 0;
}

/* Rank r's view of one token's routing (its k expert ids and weights), written to
 * receive row s: every slot j keeps its place; an expert on r becomes its rank-local
 * id with its weight, any other slot becomes -1 with weight +0.0f. The row also
 * records its source token. */
static void route_view(const int64_t *idx_row, const float *w_row, int32_t src, int k, int E,
                       int experts_per_rank, int r, int64_t s, int64_t *recv_idx, float *recv_w,
                       int32_t *recv_src)
{
    for (int j = 0; j < k; ++j) {
        int64_t e = idx_row[j];
        int64_t local = -1;
        if (e >= 0 && e < E && e / experts_per_rank == r)
            local = e - (int64_t)r * experts_per_rank;
        recv_idx[s * k + j] = local;
        recv_w[s * k + j] = local >= 0 ? w_row[j] : 0.0f;
    }
    recv_src[s] = src;
}

/* Dispatch permute: each token's row goes, unchanged, to every rank that holds
 * one of its experts, with that rank's view of the top-k routing. */
int oracle_dispatch(const uint16_t *x, const int64_t *topk_idx, const float *topk_w,
                    int64_t T, int H, int k, int E, int R, const int32_t *token_slot,
                    int64_t cap, uint16_t *recv_x, int64_t *recv_idx, float *recv_w,
                    int32_t *recv_src)
{
    if (T < 0 || H < 1 || k < 1 || E < 1 || R < 1 || E % R != 0)
        return -1;
    const int experts_per_rank = E / R;
    for (int64_t t = 0; t < T; ++t)
        for (int r = 0; r < R; ++r) {
            int64_t s = token_slot[t * R + r];
            if (s < 0)
                continue;
            if (s >= cap)
                return -1;
            memcpy(recv_x + s * H, x + t * H, (size_t)H * sizeof(uint16_t));
            route_view(topk_idx + t * k, topk_w + t * k, (int32_t)t, k, E, experts_per_rank, r, s,
                       recv_idx, recv_w, recv_src);
        }
    return 0;
}

/* FP8 dispatch: the bf16 dispatch with each row replaced by its e4m3 codes and scales. */
int oracle_dispatch_fp8(const uint16_t *x, const int64_t *topk_idx, const float *topk_w,
                        int64_t T, int H, int k, int E, int R, const int32_t *token_slot,
                        int64_t cap, uint8_t *recv_codes, float *recv_scales,
                        int64_t *recv_idx, float *recv_w, int32_t *recv_src)
{
    if (T < 0 || H < 128 || H % 128 != 0 || k < 1 || E < 1 || R < 1 || E % R != 0)
        return -1;
    const int G = H / 128;
    const int experts_per_rank = E / R;
    uint8_t *codes = (uint8_t *)malloc((size_t)(T > 0 ? T : 1) * H);
    float *scales = (float *)malloc((size_t)(T > 0 ? T : 1) * G * sizeof(float));
    if (!codes || !scales) {
        free(codes);
        free(scales);
        return -1;
    }
    oracle_quantize_fp8(x, T, H, codes, scales);
    int rc = 0;
    for (int64_t t = 0; t < T && rc == 0; ++t)
        for (int r = 0; r < R; ++r) {
            int64_t s = token_slot[t * R + r];
            if (s < 0)
                continue;
            if (s >= cap) {
                rc = -1;
                break;
            }
            memcpy(recv_codes + s * H, codes + t * H, (size_t)H);
            memcpy(recv_scales + s * G, scales + t * G, (size_t)G * sizeof(float));
            route_view(topk_idx + t * k, topk_w + t * k, (int32_t)t, k, E, experts_per_rank, r, s,
                       recv_idx, recv_w, recv_src);
        }
    free(codes);
    free(scales);
    return rc;
}

/* Packed row of (t, n) in node n's block: the number of earlier tokens with a
 * destination rank on node n; -1 when t has none there. */
int oracle_node_slots(const int64_t *topk_idx, int64_t T, int k, int E, int R, int N,
                      int32_t *node_slot)
{
    if (T < 0 || k < 1 || E < 1 || R < 1 || N < 1 || E % R != 0 || R % N != 0)
        return -1;
    const int experts_per_node = E / N;
    int32_t *filled = (int32_t *)calloc((size_t)N, sizeof(int32_t));
    uint8_t *on = (uint8_t *)malloc((size_t)N);
    if (!filled || !on) {
        free(filled);
        free(on);
        return -1;
    }
    for (int64_t t = 0; t < T; ++t) {
        memset(on, 0, (size_t)N);
        for (int j = 0; j < k; ++j) {
            const int64_t e = topk_idx[t * k + j];
            if (e >= 0 && e < E)
                on[e / experts_per_node] = 1;
        }
        for (int n = 0; n < N; ++n)
            node_slot[t * N + n] = on[n] ? filled[n]++ : -1;
    }
    free(filled);
    free(on);
    return 0;
}

/* Sparse restripe: out[n][node_slot[t][n]][p] = prob[t][n][p] for routed (t, n). */
int oracle_restripe_prob_sparse(const uint32_t *prob, int64_t T, int N, int P,
                                const int32_t *node_slot, int64_t Tmax, uint32_t *out)
{
    if (T < 0 || N < 1 || P < 1 || Tmax < T)
        return -1;
    for (int64_t t = 0; t < T; ++t)
        for (int n = 0; n < N; ++n) {
            const int64_t s = node_slot[t * N + n];
            if (s < 0)
                continue;
            if (s >= Tmax)
                return -1;
            for (int p = 0; p < P; ++p)
                out[((int64_t)n * Tmax + s) * P + p] = prob[(t * N + n) * P + p];
        }
    return 0;
}

/* Expert-major row of every (token, slot): the expert's exclusive offset plus the
 * number of earlier (token, slot) pairs, in token-then-slot order, naming the same
 * expert; -1 for masked or out-of-range ids. */
int oracle_expert_slots(const int64_t *topk_idx, int64_t T, int k, int E, int32_t *expert_slot)
{
    if (T < 0 || k < 1 || E < 1)
        return -1;
    int32_t *offset = (int32_t *)calloc((size_t)E + 1, sizeof(int32_t));
    int32_t *filled = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    if (!offset || !filled) {
        free(offset);
        free(filled);
        return -1;
    }
    for (int64_t i = 0; i < T * k; ++i)
        if (topk_idx[i] >= 0 && topk_idx[i] < E)
            offset[topk_idx[i] + 1] += 1;
    for (int e = 0; e < E; ++e)
        offset[e + 1] += offset[e];
    for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            const int64_t e = topk_idx[t * k + j];
            if (e < 0 || e >= E) {
                expert_slot[t * k + j] = -1;
                continue;
            }
            expert_slot[t * k + j] = offset[e] + filled[e];
            filled[e] += 1;
        }
    free(offset);
    free(filled);
    return 0;
}

/* Dispatch + permute: row expert_slot[t][j] = row t of x, with weight w[t][j] and
 * source token t. */
int oracle_dispatch_permute(const uint16_t *x, const int64_t *topk_idx, const float *topk_w,
                            int64_t T, int H, int k, const int32_t *expert_slot, int64_t cap,
                            uint16_t *perm_x, float *perm_w, int32_t *perm_src)
{
    (void)topk_idx;
    if (T < 0 || H < 1 || k < 1)
        return -1;
    for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            const int64_t q = expert_slot[t * k + j];
            if (q < 0)
                continue;
            if (q >= cap)
                return -1;
            memcpy(perm_x + q * H, x + t * H, (size_t)H * sizeof(uint16_t));
            perm_w[q] = topk_w[t * k + j];
            perm_src[q] = (int32_t)t;
        }
    return 0;
}

/* restripe_prob ("[PR #634] Hybrid ep nixl restripe", section "Fix"): slice
 * (t, n) of the token-major prob moves to row t of node n's block. Rows
 * T..Tmax-1 of each block are left untouched. Words are copied as bits. */
int oracle_restripe_prob(const uint32_t *prob, int64_t T, int N, int P, int64_t Tmax,
                         uint32_t *out)
{
    if (T < 0 || N < 1 || P < 1 || Tmax < T)
        return -1;
    for (int64_t t = 0; t < T; ++t)
        for (int n = 0; n < N; ++n)
            for (int p = 0; p < P; ++p)
                out[((int64_t)n * Tmax + t) * P + p] = prob[(t * N + n) * P + p];
    return 0;
}

/* Combine: out[t] = bf16( sum over ranks r = 0..R-1 holding t of partial[slot(t,r)] ),
 * summed in fp32 in ascending r starting from +0.0f. */
int oracle_combine(const uint16_t *partial, int64_t rows, const int32_t *token_slot,
                   int64_t T, int H, int R, uint16_t *out)
{
    if (T < 0 || H < 1 || R < 1)
        return -1;
    float *acc = (float *)malloc((size_t)H * sizeof(float));
    if (!acc)
        return -1;
    for (int64_t t = 0; t < T; ++t) {
        for (int h = 0; h < H; ++h)
            acc[h] = 0.0f;
        for (int r = 0; r < R; ++r) {
            int64_t s = token_slot[t * R + r];
            if (s < 0)
                continue;
            if (s >= rows) {
                free(acc);
                return -1;
            }
            for (int h = 0; h < H; ++h)
                acc[h] = acc[h] + oracle_bf16_to_f32(partial[s * H + h]);
        }
        for (int h = 0; h < H; ++h)
            out[t * H + h] = oracle_f32_to_bf16(acc[h]);
    }
    free(acc);
    return 0;
}

/* Two-phase ("hook") dispatch, "[PR #347] Feature/sm free normal kernel", section 2.1:
 * the send phase only moves data into a large per-node buffer that holds a whole batch
 * (section 2.2.2); the receive phase, called later, forwards the rows to the node's
 * ranks (the intra-node hop, section 3.3.2).
 *
 * Send: each token's row, its k expert ids and weights and its token id go once to
 * every node holding one of its experts, at row node_slot[t][n] of node n's block of
 * Tmax rows. Rows past a node's count are left untouched. */
int oracle_hook_dispatch_send(const uint16_t *x, const int64_t *topk_idx, const float *topk_w,
                              int64_t T, int H, int k, int N, const int32_t *node_slot,
                              int64_t Tmax, uint16_t *stage_x, int64_t *stage_idx,
                              float *stage_w, int32_t *stage_src)
{
    if (T < 0 || H < 1 || k < 1 || N < 1 || Tmax < 0)
        return -1;
    for (int64_t t = 0; t < T; ++t)
        for (int n = 0; n < N; ++n) {
            const int64_t ns = node_slot[t * N + n];
            if (ns < 0)
                continue;
            if (ns >= Tmax)
                return -1;
            const int64_t q = (int64_t)n * Tmax + ns;
            memcpy(stage_x + q * H, x + t * H, (size_t)H * sizeof(uint16_t));
            for (int j = 0; j < k; ++j) {
                stage_idx[q * k + j] = topk_idx[t * k + j];
                stage_w[q * k + j] = topk_w[t * k + j];
            }
            stage_src[q] = (int32_t)t;
        }
    return 0;
}

/* Receive: for each node n and each of its count_n[n] staged rows, the staged token t
 * goes to every rank r of node n with a receive slot token_slot[t][r], with rank r's
 * view of the staged routing. Together with the send phase this is the one-call
 * dispatch. */
int oracle_hook_dispatch_recv(const uint16_t *stage_x, const int64_t *stage_idx,
                              const float *stage_w, const int32_t *stage_src,
                              const int32_t *count_n, int N, int64_t Tmax, int H, int k, int E,
                              int R, const int32_t *token_slot, int64_t T, int64_t cap,
                              uint16_t *recv_x, int64_t *recv_idx, float *recv_w,
                              int32_t *recv_src)
{
    if (H < 1 || k < 1 || E < 1 || R < 1 || N < 1 || E % R != 0 || R % N != 0 || Tmax < 0)
        return -1;
    const int experts_per_rank = E / R;
    const int ranks_per_node = R / N;
    for (int n = 0; n < N; ++n) {
        if (count_n[n] < 0 || count_n[n] > Tmax)
            return -1;
        for (int64_t ns = 0; ns < count_n[n]; ++ns) {
            const int64_t q = (int64_t)n * Tmax + ns;
            const int64_t t = stage_src[q];
            if (t < 0 || t >= T)
                return -1;
            for (int r = n * ranks_per_node; r < (n + 1) * ranks_per_node; ++r) {
                const int64_t s = token_slot[t * R + r];
                if (s < 0)
                    continue;
                if (s >= cap)
                    return -1;
                memcpy(recv_x + s * H, stage_x + q * H, (size_t)H * sizeof(uint16_t));
                route_view(stage_idx + q * k, stage_w + q * k, (int32_t)t, k, E,
                           experts_per_rank, r, s, recv_idx, recv_w, recv_src);
            }
        }
    }
    return 0;
}

/* Two-phase combine (same page, sections 2.1 and 3.3.2: the send phase of combine is
 * the intra-node hop). Send: for each token t and node n with a staged row, the fp32
 * sum, from +0.0f in ascending rank order, of the partial rows of t on node n's ranks,
 * rounded once to bf16 (the element type the pages' combine moves) into row
 * node_slot[t][n] of node n's block. */
int oracle_hook_combine_send(const uint16_t *partial, int64_t rows, const int32_t *token_slot,
                             int64_t T, int H, int R, int N, const int32_t *node_slot,
                             int64_t Tmax, uint16_t *stage)
{
    if (T < 0 || H < 1 || R < 1 || N < 1 || R % N != 0 || Tmax < 0)
        return -1;
    const int ranks_per_node = R / N;
    float *sum = (float *)malloc((size_t)H * sizeof(float));
    if (!sum)
        return -1;
    for (int64_t t = 0; t < T; ++t)
        for (int n = 0; n < N; ++n) {
            const int64_t ns = node_slot[t * N + n];
            if (ns < 0)
                continue;
            if (ns >= Tmax) {
                free(sum);
                return -1;
            }
            for (int h = 0; h < H; ++h)
                sum[h] = 0.0f;
            for (int r = n * ranks_per_node; r < (n + 1) * ranks_per_node; ++r) {
                const int64_t s = token_slot[t * R + r];
                if (s < 0)
                    continue;
                if (s >= rows) {
                    free(sum);
                    return -1;
                }
                for (int h = 0; h < H; ++h)
                    sum[h] = sum[h] + oracle_bf16_to_f32(partial[s * H + h]);
            }
            const int64_t q = (int64_t)n * Tmax + ns;
            for (int h = 0; h < H; ++h)
                stage[q * H + h] = oracle_f32_to_bf16(sum[h]);
        }
    free(sum);
    return 0;
}

/* Receive: out[t] = bf16( fp32 sum, from +0.0f in ascending node order, of the staged
 * rows node_slot[t][n] of every node n holding t ); +0 for a token on no node. */
int oracle_hook_combine_recv(const uint16_t *stage, int N, int64_t Tmax,
                             const int32_t *node_slot, int64_t T, int H, uint16_t *out)
{
    if (T < 0 || H < 1 || N < 1 || Tmax < 0)
        return -1;
    float *sum = (float *)malloc((size_t)H * sizeof(float));
    if (!sum)
        return -1;
    for (int64_t t = 0; t < T; ++t) {
        for (int h = 0; h < H; ++h)
            sum[h] = 0.0f;
        for (int n = 0; n < N; ++n) {
            const int64_t ns = node_slot[t * N + n];
            if (ns < 0)
                continue;
            if (ns >= Tmax) {
                free(sum);
                return -1;
            }
            const int64_t q = (int64_t)n * Tmax + ns;
            for (int h = 0; h < H; ++h)
                sum[h] = sum[h] + oracle_bf16_to_f32(stage[q * H + h]);
        }
        for (int h = 0; h < H; ++h)
            out[t * H + h] = oracle_f32_to_bf16(sum[h]);
    }
    free(sum);
    return 0;
}
