/* ep.h -- C ABI of the single-GPU core of MoE expert-parallel (EP) dispatch/combine,
 * implemented by hand-written HIP kernels for AMD Instinct MI355X (gfx950).
 *
 * The path has four steps, after the DeepEP pull-request pages:
 *   ep_get_layout     per-rank / per-node / per-expert token counts, the token-in-rank
 *                     bitmap, exclusive prefix offsets and every (token, rank) receive slot
 *                     ("[PR #347] Feature/sm free normal kernel" names get_dispatch_layout in
 *                     its commit list; "[PR #634] Hybrid ep nixl restripe" names the scan
 *                     over tokens per local expert in its commit list);
 *   ep_dispatch       each token's bf16 row and its rank-local top-k view copied, in
 *                     ascending token order, into destination-major receive rows, one block
 *                     of rows per simulated EP rank (the intra-node copy hop of
 *                     "[PR #347]", section 3.3.2; "[PR #453] Higher Performance with Lower
 *                     SM Occupancy through Zero-Copy and TMA Offloading": data written
 *                     straight to its final buffer);
 *   ep_restripe_prob  prob [T][N][P] -> [N][Tmax][P] ("[PR #634]", sections "Baseline
 *                     problem" and "Fix");
 *   ep_combine        per token, the sum of its per-rank partial rows in fp32, rounded once
 *                     to bf16.
 * and, after the same pages, four variants of those steps:
 *   ep_dispatch_fp8          the dispatch with an e4m3 payload and one fp32 scale per 128
 *                            channels ("[PR #347]", section 3.2.1 FP8 columns);
 *   ep_dispatch_permute      the dispatch straight into expert-major rows (with the
 *                            layout's expert_slot; "[PR #634]", "dispatch+permute");
 *   ep_restripe_prob_sparse  only routed (token, node) prob slices, packed per node (with
 *                            the layout's node_slot; "[PR #634]", section "Fix");
 *   ep_dispatch_send/_recv, ep_combine_send/_recv
 *                            the two-phase ("hook") form of dispatch and combine
 *                            ("[PR #347]", sections 2.1, 2.2.2 and 3.3.2).
 *
 * Conventions for every entry point:
 *  - Every array argument is a DEVICE pointer owned by the caller; the library allocates
 *    nothing and keeps no state between calls. All arrays are dense and row-major.
 *  - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued on it and the
 *    call returns without waiting; nothing inside synchronises with the host.
 *  - Arguments are checked on the host before anything is enqueued. On any error return
 *    nothing has been enqueued. No C++ exception crosses this boundary.
 *  - Simulated topology: expert e lives on rank e / (E/R); rank r lives on node r / (R/N).
 *  - `error_flag` is one int32 in device memory. ep_get_layout overwrites it (0 or
 *    EP_DEVERR_TOPK_RANGE); every other call ORs further EP_DEVERR_* bits into it (where
 *    it is nullable, NULL drops them). After an error bit is set the affected outputs are
 *    as documented per call.
 *  - Calls that share output or workspace memory must not overlap in time.
 */
#ifndef EP_H
#define EP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    EP_OK = 0,
    EP_ERR_ARG = -1,       /* a count or size out of range, or a required pointer is NULL */
    EP_ERR_ALIGN = -2,     /* a pointer or row length breaks the alignment rule of the call */
    EP_ERR_CAPACITY = -3,  /* a destination or workspace smaller than the call requires
                              (the host-side counterpart of the check against too large a
                              receive token count in the commit list of "[PR #453] Higher
                              Performance with Lower SM Occupancy through Zero-Copy and TMA
                              Offloading") */
    EP_ERR_HIP = -4        /* the HIP runtime reported an error when the work was enqueued */
};

/* Bits the kernels OR into *error_flag. */
#define EP_DEVERR_TOPK_RANGE    1  /* a topk_idx entry < -1 or >= num_experts (entry skipped) */
#define EP_DEVERR_RECV_OVERFLOW 2  /* a destination row past its buffer: a slot >= the receive
                                      capacity, a node slot >= Tmax, a node count above
                                      min(T, Tmax) (row skipped) */
#define EP_DEVERR_SLOT_RANGE    4  /* a source row out of range: a slot >= num_partial_rows, a
                                      staged token outside [0, T), a node slot >= Tmax in
                                      ep_combine_recv (skipped) */
#define EP_DEVERR_WORKSPACE     8  /* ep_layout_counts found its workspace's ticket not zero
                                      on entry (outputs of that call and of the
                                      ep_dispatch_layout after it are unspecified) */

/* Limits of this implementation. */
#define EP_MAX_RANKS   1024
#define EP_MAX_EXPERTS 8192
#define EP_EXPERT_SLOT_MAX_K 16  /* largest top-k for which ep_get_layout fills expert_slot */
#define EP_LAYOUT_SCRATCH_BYTES 4194304  /* device scratch of ep_get_layout_no_alloc (4 MiB) */
#define EP_COUNTS_MAX_RANKS 64  /* largest num_ranks of ep_layout_counts / ep_dispatch_layout */
#define EP_LAYOUT_DISPATCH_MAX_TOKENS 256  /* largest batch of ep_layout_dispatch */

/* Static string for a status code; never NULL. */
const char *ep_status_string(int status);

/* Bytes of device workspace ep_get_layout needs for these sizes: the size query a caller
 * makes before allocating ("[PR #347] Feature/sm free normal kernel", section 2.2.2, a
 * utility that estimates the minimum buffer size before the call). The workspace holds
 * per-256-token-block count tables: rank counts [nb][R], node counts [nb][N], two expert
 * tables [nb][E] and error bits [nb], nb = ceil(T / 256), each 256-byte aligned; for 2 to
 * 16 blocks at num_ranks <= EP_COUNTS_MAX_RANKS, at least ep_layout_counts_workspace_bytes
 * (such a batch, when no node or expert slots are asked for, is counted as the counts path
 * counts it). Returns 0 when num_tokens == 0 (no workspace needed; NULL is then accepted)
 * and also when the sizes are ones ep_get_layout rejects. */
size_t ep_layout_workspace_bytes(int64_t num_tokens, int num_experts, int num_ranks,
                                 int num_nodes);

/* ep_get_layout -- the dispatch layout of one batch.
 *
 * In:  topk_idx      int64 [T][k]; expert id per (token, slot); -1 marks an unused slot.
 * Out (all int32 unless noted; NULL allowed where marked):
 *   num_tokens_per_rank    [R]    tokens with at least one expert on rank r (a token counts
 *                                 once per rank however many of its experts the rank holds)
 *   num_tokens_per_node    [N]    tokens with at least one expert on node n       (nullable)
 *   num_tokens_per_expert  [E]    (token, slot) pairs naming expert e             (nullable)
 *   is_token_in_rank uint8 [T][R] 1 if token t has an expert on rank r, else 0    (nullable)
 *   rank_offset            [R+1]  exclusive prefix sum of num_tokens_per_rank; rank_offset[R]
 *                                 = M, the number of (token, rank) pairs
 *   expert_offset          [E+1]  exclusive prefix sum of num_tokens_per_expert   (nullable)
 *   token_slot             [T][R] receive row of (t, r) = rank_offset[r] + number of tokens
 *                                 t' < t on rank r; -1 where t is not on r. The rows of rank
 *                                 r are rank_offset[r] .. rank_offset[r+1]-1, in token order.
 *   expert_slot            [T][k] expert-major row of (t, j) for ep_dispatch_permute:
 *                                 expert_offset[e] + the number of earlier pairs, in
 *                                 (token, slot) order, naming the same expert e; -1 for a
 *                                 masked or bad id. Rank r's experts are one contiguous range
 *                                 of rows. Needs k <= EP_EXPERT_SLOT_MAX_K.       (nullable)
 *   node_slot              [T][N] packed row of (t, n) for ep_restripe_prob_sparse: the
 *                                 number of tokens t' < t with a destination on node n; -1
 *                                 where t has none on n.                          (nullable)
 *   error_flag             [1]    overwritten: 0, or EP_DEVERR_TOPK_RANGE when an entry is
 *                                 < -1 or >= E (such entries are skipped like -1).
 * Workspace: `workspace` of `workspace_bytes` >= ep_layout_workspace_bytes(T, E, R, N) bytes,
 *   16-byte aligned, contents on entry irrelevant, clobbered.
 * Sizes: T >= 0, 1 <= k <= E, 1 <= R <= EP_MAX_RANKS, E <= EP_MAX_EXPERTS, E % R == 0,
 *   1 <= N, R % N == 0, T * min(k, R) <= INT32_MAX; and T * k <= INT32_MAX when any of
 *   num_tokens_per_expert, expert_offset or expert_slot is non-NULL (they count
 *   (token, slot) pairs in int32).
 * Errors: EP_ERR_ARG (sizes, NULL), EP_ERR_ALIGN (int32/int64 arrays not naturally aligned,
 *   workspace not 16-byte aligned), EP_ERR_CAPACITY (workspace too small), EP_ERR_HIP.
 * T == 0 is valid: counts and offsets are written as zeros. */
int ep_get_layout(const int64_t *topk_idx, int64_t num_tokens, int num_topk,
                  int num_experts, int num_ranks, int num_nodes,
                  int32_t *num_tokens_per_rank, int32_t *num_tokens_per_node,
                  int32_t *num_tokens_per_expert, uint8_t *is_token_in_rank,
                  int32_t *rank_offset, int32_t *expert_offset, int32_t *token_slot,
                  int32_t *expert_slot, int32_t *node_slot, int32_t *error_flag,
                  void *workspace, size_t workspace_bytes, void *stream);

/* ep_get_layout_no_alloc -- ep_get_layout for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments, checks and outputs, bit for bit, but no workspace argument. The
 * per-block count tables live in a static device array of EP_LAYOUT_SCRATCH_BYTES that
 * the library holds on each GPU it runs on until the process ends; this call makes no
 * allocation of any kind.
 * Limit: ep_layout_workspace_bytes(T, E, R, N) <= EP_LAYOUT_SCRATCH_BYTES, else
 *   EP_ERR_CAPACITY with nothing enqueued (at E = 256, R = 64, N = 8: up to 458 752
 *   tokens).
 * Every call on one GPU shares that GPU's array, and it keeps the last call's contents
 * (nothing in it needs to start at zero). Calls whose work overlaps in time on one GPU --
 * on two streams, or from two threads -- race on the array and give undefined outputs;
 * stream-ordered calls are safe.
 * `stream` must belong to the current device (else EP_ERR_ARG). The first call on a
 * device looks up that device's address of the array (EP_ERR_HIP if the lookup fails).
 * Errors: as ep_get_layout, with EP_ERR_CAPACITY for sizes past the scratch. */
int ep_get_layout_no_alloc(const int64_t *topk_idx, int64_t num_tokens, int num_topk,
                           int num_experts, int num_ranks, int num_nodes,
                           int32_t *num_tokens_per_rank, int32_t *num_tokens_per_node,
                           int32_t *num_tokens_per_expert, uint8_t *is_token_in_rank,
                           int32_t *rank_offset, int32_t *expert_offset, int32_t *token_slot,
                           int32_t *expert_slot, int32_t *node_slot, int32_t *error_flag,
                           void *stream);

/* ep_dispatch_preprocess -- ep_get_layout and ep_restripe_prob of the same batch in one
 * call: the preprocessing a dispatch needs before it moves rows ("[PR #634] Hybrid ep nixl
 * restripe", section "Fix": the restripe is part of the dispatch's preprocessing, in place
 * of the copy it replaces there). Outputs are exactly those of the two calls: the layout
 * outputs as ep_get_layout with the same arguments, and prob_dest_major as
 * ep_restripe_prob(prob, T, num_nodes, prob_per_token, max_tokens_per_rank). The
 * restripe's blocks run inside the layout's first kernel launch, after the layout's own
 * blocks, so the pair costs one launch less than the two calls.
 * Sizes and errors: those of both calls (EP_ERR_CAPACITY also for Tmax < T). */
int ep_dispatch_preprocess(const int64_t *topk_idx, int64_t num_tokens, int num_topk,
                           int num_experts, int num_ranks, int num_nodes,
                           int32_t *num_tokens_per_rank, int32_t *num_tokens_per_node,
                           int32_t *num_tokens_per_expert, uint8_t *is_token_in_rank,
                           int32_t *rank_offset, int32_t *expert_offset, int32_t *token_slot,
                           int32_t *expert_slot, int32_t *node_slot, int32_t *error_flag,
                           const float *prob, int prob_per_token, int64_t max_tokens_per_rank,
                           float *prob_dest_major, void *workspace, size_t workspace_bytes,
                           void *stream);

/* The counts path: the layout and the dispatch in two kernel launches instead of three, for
 * num_ranks <= EP_COUNTS_MAX_RANKS. ep_get_layout needs a launch to count and one to turn
 * the counts into every (token, rank) receive row ("[PR #347] Feature/sm free normal kernel"
 * names get_dispatch_layout before the dispatch in its commit list). Here the second of
 * those launches is folded into the dispatch: ep_layout_counts counts per 256-token block
 * into the workspace (and may restripe prob in the same launch, as ep_dispatch_preprocess
 * does); ep_dispatch_layout computes each token's receive rows inside the dispatch's waves
 * from those tables, writing token_slot and the bitmap as it goes, and the rank, node and
 * expert counts and offsets in a few blocks of its own. Together the two calls give every
 * output of ep_get_layout (without node_slot and expert_slot), ep_restripe_prob and
 * ep_dispatch, bit for bit. error_flag is overwritten by ep_layout_counts (0, or
 * EP_DEVERR_TOPK_RANGE) and only ORed into by ep_dispatch_layout.
 *
 * Workspace: `workspace` of at least ep_layout_counts_workspace_bytes(T, E, R, N) bytes,
 *   16-byte aligned. Its first 4 bytes are a ticket counter that must be ZERO before the
 *   first call (say hipMemset once after allocation); every call of ep_layout_counts leaves
 *   it zero again (EP_DEVERR_WORKSPACE reports a non-zero one in a batch of more than 4096
 *   tokens; smaller batches do not use it). The rest is rewritten by every call. Use it for
 *   nothing else, pass the same one (with the same T, E, R, N) to ep_dispatch_layout, and
 *   do not let calls on one workspace overlap in time.
 * Returns 0 for sizes ep_layout_counts rejects. */
size_t ep_layout_counts_workspace_bytes(int64_t num_tokens, int num_experts, int num_ranks,
                                        int num_nodes);

/* ep_layout_counts -- In: topk_idx int64 [T][k]. Out: the per-block tables in `workspace`,
 * error_flag [1] (overwritten); with expert_rank non-NULL ([T][k] int32, k <=
 * EP_EXPERT_SLOT_MAX_K), each pair's rank among the pairs of its block of 256 tokens that
 * name the same expert, in (token, slot) order (-1 for a masked or bad id), for
 * ep_dispatch_permute_layout. With prob non-NULL it also writes prob_dest_major exactly
 * as ep_restripe_prob(prob, T, num_nodes, prob_per_token, max_tokens_per_rank).
 * Sizes: as ep_get_layout, num_ranks <= EP_COUNTS_MAX_RANKS and T * k <= INT32_MAX; with
 *   prob as ep_restripe_prob (EP_ERR_CAPACITY for Tmax < T).
 * Errors: EP_ERR_ARG, EP_ERR_ALIGN, EP_ERR_CAPACITY (workspace too small or NULL),
 *   EP_ERR_HIP. */
int ep_layout_counts(const int64_t *topk_idx, int64_t num_tokens, int num_topk, int num_experts,
                     int num_ranks, int num_nodes, int32_t *error_flag, int32_t *expert_rank,
                     const float *prob, int prob_per_token, int64_t max_tokens_per_rank,
                     float *prob_dest_major, void *workspace, size_t workspace_bytes,
                     void *stream);

/* ep_dispatch_layout -- after ep_layout_counts on the same batch and workspace, stream-
 * ordered: ep_dispatch's outputs (recv_x, recv_topk_idx, recv_topk_weights, recv_src_idx,
 * with the same meaning, capacity rule and error bits) and ep_get_layout's token_slot
 * [T][R], and, nullable, num_tokens_per_rank [R], rank_offset [R+1], is_token_in_rank
 * [T][R], num_tokens_per_node [N], num_tokens_per_expert [E] and expert_offset [E+1], all
 * as ep_get_layout defines them. topk_idx is required.
 * Sizes: as ep_dispatch, num_ranks <= EP_COUNTS_MAX_RANKS, num_nodes as given to
 *   ep_layout_counts. Errors: EP_ERR_ARG, EP_ERR_ALIGN, EP_ERR_CAPACITY (workspace),
 *   EP_ERR_HIP. */
int ep_dispatch_layout(const void *x, const int64_t *topk_idx, const float *topk_weights,
                       int64_t num_tokens, int hidden, int num_topk, int num_experts,
                       int num_ranks, int num_nodes, int32_t *num_tokens_per_rank,
                       int32_t *rank_offset, int32_t *num_tokens_per_node,
                       int32_t *num_tokens_per_expert, int32_t *expert_offset,
                       int32_t *token_slot, uint8_t *is_token_in_rank, void *recv_x,
                       int64_t *recv_topk_idx, float *recv_topk_weights, int32_t *recv_src_idx,
                       int64_t recv_capacity, int32_t *error_flag, const void *workspace,
                       size_t workspace_bytes, void *stream);

/* ep_layout_dispatch -- the layout, the dispatch and (with prob) the restripe of a batch of
 * at most EP_LAYOUT_DISPATCH_MAX_TOKENS tokens in one kernel launch, so that a decode-sized
 * step is this call and ep_combine. It computes get_dispatch_layout and then the dispatch
 * ("[PR #347] Feature/sm free normal kernel": commit list, and section 3.2.1 for the
 * dispatch's payload) and the restripe that replaces dispatch_preprocess's copy ("[PR #634]
 * Hybrid ep nixl restripe", section "Fix"). Outputs, bit for bit those of ep_get_layout +
 * ep_dispatch (+ ep_restripe_prob) with the same meanings: num_tokens_per_rank [R],
 * rank_offset [R+1], token_slot [T][R] and recv_x (all required when T > 0);
 * is_token_in_rank [T][R], num_tokens_per_node [N], num_tokens_per_expert [E],
 * expert_offset [E+1], recv_topk_idx, recv_topk_weights, recv_src_idx (nullable); with
 * prob non-NULL, prob_dest_major as ep_restripe_prob(prob, T, num_nodes, prob_per_token,
 * max_tokens_per_rank). error_flag [1] is overwritten: 0, or EP_DEVERR_TOPK_RANGE and
 * EP_DEVERR_RECV_OVERFLOW as ep_get_layout and ep_dispatch set them (rows past
 * recv_capacity are skipped). Each block of the launch recomputes the batch's rank masks
 * from topk_idx, so no block waits for another.
 * Sizes: 0 <= T <= EP_LAYOUT_DISPATCH_MAX_TOKENS, num_ranks <= EP_COUNTS_MAX_RANKS, the
 *   rest as ep_get_layout and ep_dispatch; with prob as ep_restripe_prob (EP_ERR_CAPACITY
 *   for Tmax < T). Errors: EP_ERR_ARG, EP_ERR_ALIGN, EP_ERR_CAPACITY, EP_ERR_HIP. */
int ep_layout_dispatch(const void *x, const int64_t *topk_idx, const float *topk_weights,
                       int64_t num_tokens, int hidden, int num_topk, int num_experts,
                       int num_ranks, int num_nodes, int32_t *num_tokens_per_rank,
                       int32_t *rank_offset, int32_t *num_tokens_per_node,
                       int32_t *num_tokens_per_expert, int32_t *expert_offset,
                       int32_t *token_slot, uint8_t *is_token_in_rank, void *recv_x,
                       int64_t *recv_topk_idx, float *recv_topk_weights, int32_t *recv_src_idx,
                       int64_t recv_capacity, const float *prob, int prob_per_token,
                       int64_t max_tokens_per_rank, float *prob_dest_major, int32_t *error_flag,
                       void *stream);

/* ep_dispatch_permute_layout -- the counts path's dispatch + permute ("[PR #634] Hybrid ep
 * nixl restripe" measures "dispatch+permute"; its commit list names the scan over tokens
 * per local expert): after ep_layout_counts on the same batch and workspace with
 * expert_rank, stream-ordered, ep_dispatch_permute's outputs (perm_x, perm_weights,
 * perm_src_idx, with the same meaning and capacity rule) for the expert-major rows that
 * ep_get_layout's expert_slot defines, computed inside the permute's waves; and, nullable,
 * expert_slot [T][k], num_tokens_per_expert [E] and expert_offset [E+1] as ep_get_layout
 * defines them. topk_idx and expert_rank are required.
 * Sizes: as ep_dispatch_permute, num_ranks <= EP_COUNTS_MAX_RANKS, and T <= 16384 (at most
 *   64 blocks of 256 tokens: each wave reads one word per block). Errors: EP_ERR_ARG,
 *   EP_ERR_ALIGN, EP_ERR_CAPACITY (workspace), EP_ERR_HIP. */
int ep_dispatch_permute_layout(const void *x, const int64_t *topk_idx,
                               const float *topk_weights, int64_t num_tokens, int hidden,
                               int num_topk, int num_experts, int num_ranks, int num_nodes,
                               const int32_t *expert_rank, int32_t *num_tokens_per_expert,
                               int32_t *expert_offset, int32_t *expert_slot, void *perm_x,
                               float *perm_weights, int32_t *perm_src_idx, int64_t perm_capacity,
                               int32_t *error_flag, const void *workspace, size_t workspace_bytes,
                               void *stream);

/* ep_dispatch -- pack every (token, rank) pair into its receive row.
 *
 * In:  x            bf16 [T][H] (any 16-bit payload; copied as bits)
 *      topk_idx     int64 [T][k], topk_weights fp32 [T][k] (may be NULL when
 *                   recv_topk_weights is NULL)
 *      token_slot   int32 [T][R] from ep_get_layout
 * Out: for each t, r with s = token_slot[t][r] >= 0:
 *      recv_x            bf16 [cap][H]  row s = row t of x
 *      recv_topk_idx     int64 [cap][k] row s, slot j = e - r*E/R if expert e = topk_idx[t][j]
 *                                       lives on r, else -1                       (nullable)
 *      recv_topk_weights fp32 [cap][k]  topk_weights[t][j] where recv_topk_idx is >= 0,
 *                                       else +0.0f                                (nullable)
 *      recv_src_idx      int32 [cap]    t                                         (nullable)
 *      Rows >= M are not written.
 * Sizes: H % 8 == 0; x and recv_x 16-byte aligned (rows move as 128-bit words);
 *   recv_capacity >= 0 rows. A slot >= recv_capacity is skipped and sets
 *   EP_DEVERR_RECV_OVERFLOW, so a capacity of T * min(k, R) never overflows and a capacity
 *   of exactly M (read back from rank_offset[R]) is also valid.
 * Errors: EP_ERR_ARG, EP_ERR_ALIGN, EP_ERR_HIP. */
int ep_dispatch(const void *x, const int64_t *topk_idx, const float *topk_weights,
                int64_t num_tokens, int hidden, int num_topk, int num_experts, int num_ranks,
                const int32_t *token_slot, void *recv_x, int64_t *recv_topk_idx,
                float *recv_topk_weights, int32_t *recv_src_idx, int64_t recv_capacity,
                int32_t *error_flag, void *stream);

/* ep_dispatch_fp8 -- ep_dispatch with an FP8 payload: each token is quantised once and
 * every destination row receives its e4m3 codes and per-128-channel scales ("[PR #347]",
 * section 3.2.1, and "[PR #453]" measure dispatch with an FP8 payload; their byte counts
 * fit one fp32 scale per 128 channels, 7168 + 224 bytes per 7168-wide row).
 *
 * In:  x            bf16 [T][H], finite values
 *      topk_idx, topk_weights, token_slot as for ep_dispatch
 * Out: for each t, r with s = token_slot[t][r] >= 0, and each group g of 128 channels:
 *      recv_scales     fp32 [cap][H/128]  scale = amax / 448, amax = max |x[t][128g .. 128g+127]|
 *                                         (1.0 for an all-zero group)
 *      recv_x_fp8      uint8 [cap][H]     OCP e4m3 (E4M3FN) code of x[t][c] * (448 / amax),
 *                                         rounded to nearest even, magnitude at most 448
 *      recv_topk_idx, recv_topk_weights, recv_src_idx as for ep_dispatch (nullable)
 *      Rows >= M are not written.
 * Sizes: H % 128 == 0; x and recv_x_fp8 16-byte aligned, recv_scales 4-byte aligned.
 *   Slots >= recv_capacity are skipped and set EP_DEVERR_RECV_OVERFLOW.
 * Errors: EP_ERR_ARG, EP_ERR_ALIGN, EP_ERR_HIP. */
int ep_dispatch_fp8(const void *x, const int64_t *topk_idx, const float *topk_weights,
                    int64_t num_tokens, int hidden, int num_topk, int num_experts,
                    int num_ranks, const int32_t *token_slot, uint8_t *recv_x_fp8,
                    float *recv_scales, int64_t *recv_topk_idx, float *recv_topk_weights,
                    int32_t *recv_src_idx, int64_t recv_capacity, int32_t *error_flag,
                    void *stream);

/* ep_dispatch_permute -- dispatch straight into expert-major rows ("[PR #634] Hybrid ep nixl
 * restripe" measures "dispatch+permute"; its commit list names the scan over tokens per
 * local expert that orders them): the rows a grouped expert GEMM consumes.
 *
 * In:  x            bf16 [T][H]
 *      topk_weights fp32 [T][k] (may be NULL when perm_weights is NULL)
 *      expert_slot  int32 [T][k] from ep_get_layout
 * Out: for each t, j with q = expert_slot[t][j] >= 0:
 *      perm_x       bf16 [cap][H]  row q = row t of x
 *      perm_weights fp32 [cap]     topk_weights[t][j]                              (nullable)
 *      perm_src_idx int32 [cap]    t                                               (nullable)
 *      Rows of expert e are expert_offset[e] .. expert_offset[e+1]-1, tokens ascending.
 * Sizes: H % 8 == 0; x and perm_x 16-byte aligned; a row >= capacity is skipped and sets
 *   EP_DEVERR_RECV_OVERFLOW (capacity T * k never overflows).
 * Errors: EP_ERR_ARG, EP_ERR_ALIGN, EP_ERR_HIP. */
int ep_dispatch_permute(const void *x, const float *topk_weights, int64_t num_tokens, int hidden,
                        int num_topk, const int32_t *expert_slot, void *perm_x,
                        float *perm_weights, int32_t *perm_src_idx, int64_t capacity,
                        int32_t *error_flag, void *stream);

/* ep_restripe_prob -- prob from token-major to destination-major
 * ("[PR #634] Hybrid ep nixl restripe", section "Fix").
 *
 * In:  prob            fp32 [T][N][P]
 * Out: prob_dest_major fp32 [N][Tmax][P]; element [n][t][p] = prob[t][n][p] for t < T, copied
 *      as 32-bit words. Rows t in [T, Tmax) of every node block are not written.
 * Sizes: T >= 0, N >= 1, P >= 1, Tmax >= T (else EP_ERR_CAPACITY). When P % 4 == 0 and both
 *   pointers are 16-byte aligned slices move as 128-bit words, otherwise as 32-bit words.
 * Errors: EP_ERR_ARG, EP_ERR_ALIGN (pointers not 4-byte aligned), EP_ERR_CAPACITY,
 *   EP_ERR_HIP. */
int ep_restripe_prob(const float *prob, int64_t num_tokens, int num_nodes, int prob_per_token,
                     int64_t max_tokens_per_rank, float *prob_dest_major, void *stream);

/* ep_restripe_prob_sparse -- the sparse-path restripe ("[PR #634]", section "Fix": one put
 * per run in the sparse path): only slices of tokens routed to a node move, packed in
 * token order at the start of the node's block, so any run of consecutive routed tokens
 * is one contiguous range.
 *
 * In:  prob        fp32 [T][N][P]
 *      node_slot   int32 [T][N] from ep_get_layout
 * Out: prob_dest_major fp32 [N][Tmax][P]; row node_slot[t][n] of block n = prob[t][n][:] for
 *      every (t, n) with node_slot[t][n] >= 0 (32-bit words copied as bits). Other rows are
 *      not written. A slot >= Tmax is skipped and sets EP_DEVERR_RECV_OVERFLOW (error_flag
 *      nullable).
 * Sizes and alignment as for ep_restripe_prob. Errors: EP_ERR_ARG, EP_ERR_ALIGN,
 *   EP_ERR_CAPACITY (Tmax < T), EP_ERR_HIP. */
int ep_restripe_prob_sparse(const float *prob, int64_t num_tokens, int num_nodes,
                            int prob_per_token, const int32_t *node_slot,
                            int64_t max_tokens_per_rank, float *prob_dest_major,
                            int32_t *error_flag, void *stream);

/* ep_combine -- gather each token's per-rank partial rows back to token order and sum them:
 * the reverse of ep_dispatch, moving the same rows back ("[PR #347] Feature/sm free normal
 * kernel", section 3.2.1: its combine table measures the dispatch payload travelling back;
 * "[PR #453]" description: combine measured beside dispatch). The sum is unweighted: the
 * top-k weights are taken to be applied inside each rank's expert output.
 *
 * In:  partial     bf16 [num_partial_rows][H], laid out like ep_dispatch's recv_x
 *      token_slot  int32 [T][R] from ep_get_layout
 * Out: out         bf16 [T][H]; out[t][h] = bf16_rne( sum over r = 0..R-1 with
 *                  s = token_slot[t][r] >= 0 of float(partial[s][h]) ), accumulated in fp32
 *                  in ascending r from +0.0f; a token on no rank gets +0.0.
 * Sizes: H % 8 == 0; partial and out 16-byte aligned. A slot >= num_partial_rows is skipped
 *   and sets EP_DEVERR_SLOT_RANGE.
 * Errors: EP_ERR_ARG, EP_ERR_ALIGN, EP_ERR_HIP. */
int ep_combine(const void *partial, int64_t num_partial_rows, const int32_t *token_slot,
               int64_t num_tokens, int hidden, int num_ranks, void *out, int32_t *error_flag,
               void *stream);

/* Two-phase ("hook") dispatch and combine ("[PR #347] Feature/sm free normal kernel",
 * section 2.1): the first call runs only the send phase and returns; the caller may run
 * other work (the page overlaps a GEMM) and later makes the receive-phase call on a
 * stream ordered after the send. Between the two, a per-node staging buffer of Tmax rows
 * per node holds the whole batch (the large buffer of section 2.2.2; on one GPU it is both
 * the send and the receive side of that buffer). The receive phase of dispatch and the
 * send phase of combine are the intra-node hop (section 3.3.2). Staged row (n, s) is row
 * n * Tmax + s of every staging array.
 *
 * The send phases take a workgroup budget, the counterpart of the page's point that hook
 * mode frees SMs for compute while the data moves (section 2.2.2; "[PR #453] Higher
 * Performance with Lower SM Occupancy through Zero-Copy and TMA Offloading" counts the SMs
 * its kernels occupy). num_workgroups == 0 launches the full grid (the fastest send when
 * it runs alone); num_workgroups > 0 launches at most that many workgroups, each looping
 * over its share of the work, so a kernel on another queue (say a GEMM) keeps room on
 * every CU. The results are the same either way. Overlap needs the two streams to feed
 * different hardware queues.
 *
 * ep_dispatch_send -- In: x bf16 [T][H]; topk_idx int64 [T][k]; topk_weights fp32 [T][k];
 *      node_slot int32 [T][N] from ep_get_layout.
 * Out: for every (t, n) with s = node_slot[t][n] >= 0, staged row (n, s):
 *      stage_x     bf16 [N][Tmax][H]  row t of x
 *      stage_topk_idx     int64 [N][Tmax][k]  topk_idx[t][:] unchanged          (nullable)
 *      stage_topk_weights fp32  [N][Tmax][k]  topk_weights[t][:] unchanged      (nullable)
 *      stage_src   int32 [N][Tmax]    t
 *      Other rows are not written. A slot >= Tmax is skipped and sets
 *      EP_DEVERR_RECV_OVERFLOW. topk_idx / topk_weights may be NULL when the matching
 *      staging array is NULL.
 * num_workgroups: 0 (full grid) or the most 256-thread workgroups to occupy.
 * Sizes: H % 8 == 0; x and stage_x 16-byte aligned. Errors: EP_ERR_ARG (also
 *   num_workgroups < 0), EP_ERR_ALIGN, EP_ERR_HIP. */
int ep_dispatch_send(const void *x, const int64_t *topk_idx, const float *topk_weights,
                     int64_t num_tokens, int hidden, int num_topk, int num_nodes,
                     const int32_t *node_slot, int64_t max_tokens_per_rank, void *stage_x,
                     int64_t *stage_topk_idx, float *stage_topk_weights, int32_t *stage_src,
                     int32_t *error_flag, int num_workgroups, void *stream);

/* ep_dispatch_recv -- In: the staging arrays written by ep_dispatch_send; count_n int32 [N]
 *      (num_tokens_per_node from ep_get_layout: the staged rows of node n are 0..count_n[n]-1);
 *      token_slot int32 [T][R] from ep_get_layout.
 * Out: exactly what ep_dispatch writes: for every staged row (n, s) with token
 *      t = stage_src[n][s] and every rank r of node n with d = token_slot[t][r] >= 0, row d
 *      of recv_x = the staged row, recv_topk_idx / recv_topk_weights [d] = rank r's view of
 *      the staged routing (local id and weight where the expert is on r, else -1 and +0.0f),
 *      recv_src_idx[d] = t. recv_topk_idx needs stage_topk_idx; recv_topk_weights needs
 *      both staged arrays. A staged token outside [0, T) sets EP_DEVERR_SLOT_RANGE; a count
 *      above min(T, Tmax) or a row >= recv_capacity sets EP_DEVERR_RECV_OVERFLOW.
 * Sizes: as ep_dispatch, and R % N == 0. Errors: EP_ERR_ARG, EP_ERR_ALIGN, EP_ERR_HIP. */
int ep_dispatch_recv(const void *stage_x, const int64_t *stage_topk_idx,
                     const float *stage_topk_weights, const int32_t *stage_src,
                     const int32_t *count_n, int num_nodes, int64_t max_tokens_per_rank,
                     int hidden, int num_topk, int num_experts, int num_ranks,
                     const int32_t *token_slot, int64_t num_tokens, void *recv_x,
                     int64_t *recv_topk_idx, float *recv_topk_weights, int32_t *recv_src_idx,
                     int64_t recv_capacity, int32_t *error_flag, void *stream);

/* ep_combine_send -- In: partial bf16 [num_partial_rows][H] (ep_dispatch's receive layout);
 *      token_slot int32 [T][R]; node_slot int32 [T][N] from ep_get_layout.
 * Out: stage bf16 [N][Tmax][H]; for every (t, n) with s = node_slot[t][n] >= 0, staged row
 *      (n, s) = bf16_rne( sum over the ranks r of node n, ascending, with
 *      d = token_slot[t][r] >= 0 of float(partial[d]) ), fp32 from +0.0f. Other rows are not
 *      written. A slot >= num_partial_rows sets EP_DEVERR_SLOT_RANGE, a node slot >= Tmax
 *      EP_DEVERR_RECV_OVERFLOW (both skipped).
 *      num_workgroups: 0 (full grid) or the most 1024-thread workgroups to occupy
 *      (EP_ERR_ARG if < 0).
 * ep_combine_recv -- In: stage from ep_combine_send; node_slot.
 * Out: out bf16 [T][H]; out[t] = bf16_rne( sum over nodes n ascending with
 *      s = node_slot[t][n] >= 0 of float(staged row (n, s)) ), fp32 from +0.0f; +0.0 for a
 *      token on no node. A node slot >= Tmax is skipped and sets EP_DEVERR_SLOT_RANGE.
 *      The result differs from ep_combine's by the extra rounding of each node's sum.
 * Sizes: H % 8 == 0; partial, stage and out 16-byte aligned; R % N == 0.
 * Errors: EP_ERR_ARG, EP_ERR_ALIGN, EP_ERR_HIP. */
int ep_combine_send(const void *partial, int64_t num_partial_rows, const int32_t *token_slot,
                    int64_t num_tokens, int hidden, int num_ranks, int num_nodes,
                    const int32_t *node_slot, int64_t max_tokens_per_rank, void *stage,
                    int32_t *error_flag, int num_workgroups, void *stream);
int ep_combine_recv(const void *stage, int num_nodes, int64_t max_tokens_per_rank,
                    const int32_t *node_slot, int64_t num_tokens, int hidden, void *out,
                    int32_t *error_flag, void *stream);

/* ep_hbm_copy -- measurement helper, not a step of the path: a plain 128-bit copy of
 * `bytes` bytes (a multiple of 16; both pointers 16-byte aligned) used as the HBM
 * copy-bandwidth yardstick and as the known-size reference for hardware byte counters.
 * Loads are non-temporal and stores device-scope (written through the L2), the fastest
 * pair measured for a copy on MI355X.
 * Errors: EP_ERR_ARG, EP_ERR_ALIGN, EP_ERR_HIP. */
int ep_hbm_copy(const void *src, void *dst, size_t bytes, void *stream);

/* ep_hbm_fan -- measurement helper, not a step of the path: the yardstick for a mix of
 * reads and writes. src holds fan_in slabs and dst fan_out slabs of slab_bytes each
 * (contiguous, slab s at byte s * slab_bytes); every output slab becomes the bitwise XOR of
 * the input slabs. fan_in F with fan_out 1 reads F bytes per byte written (the direction
 * mix of ep_combine), fan_in 1 with fan_out F the reverse (that of ep_dispatch); all
 * accesses are sequential 128-bit streams, with cached loads and stores that are
 * non-temporal at device scope when fan_in < fan_out (as the dispatch's rows), and
 * non-temporal loads and stores otherwise. slab_bytes a multiple of 16,
 * both pointers 16-byte aligned, 1 <= fan_in, fan_out <= 64.
 * Errors: EP_ERR_ARG, EP_ERR_ALIGN, EP_ERR_HIP. */
int ep_hbm_fan(const void *src, void *dst, size_t slab_bytes, int fan_in, int fan_out,
               void *stream);

/* ep_hbm_spread -- measurement helper, not a step of the path: the fan-in yardstick with
 * its reads spread over `regions` sequential streams, as the combine's source rows lie in
 * one block of the receive buffer per rank. dst is cut into chunks of
 * EP_HBM_SPREAD_CHUNK_BYTES; src holds fan_in * out_bytes bytes cut into `regions` equal
 * regions, back to back. Output chunk b becomes the bitwise XOR of the input chunks
 * j = fan_in * b + q (0 <= q < fan_in), chunk j being chunk j / regions of region
 * j % regions, so each region is read from its start in order. Loads and stores are
 * non-temporal. out_bytes a multiple of EP_HBM_SPREAD_CHUNK_BYTES, 1 <= fan_in <= 8,
 * 1 <= regions <= EP_MAX_RANKS, (fan_in * out_bytes / EP_HBM_SPREAD_CHUNK_BYTES) % regions
 * == 0 (else EP_ERR_ARG); both pointers 16-byte aligned.
 * Errors: EP_ERR_ARG, EP_ERR_ALIGN, EP_ERR_HIP. */
#define EP_HBM_SPREAD_CHUNK_BYTES 4096
int ep_hbm_spread(const void *src, void *dst, size_t out_bytes, int fan_in, int regions,
                  void *stream);

#ifdef __cplusplus
}
#endif

#endif /* EP_H */
