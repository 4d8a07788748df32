/*
 * fa.h -- C ABI of libfa.so: exact, IO-aware, tiled attention forward (and
 * its key-split variant and backward) on MI355X (gfx950).
 *
 * What it computes. For every batch b, query head h and query row i, with kv
 * head g = h / (H / H_kv) and visible keys V_i = { j < T : !causal or j <= i }:
 *   s_ij = scale * q[b,i,h,:] . k[b,j,g,:]
 *   o[b,i,h,:] = sum_{j in V_i} softmax_j(s_i.) * v[b,j,g,:]
 *   lse[b,h,i] = ln sum_{j in V_i} exp(s_ij)
 * in one fused kernel: the T x T score matrix never reaches device memory.
 * This is the forward pass described by
 *  - "Flash Attention Memory Optimization Explained" (lzwjava.github.io),
 *    sections "What is Flash Attention?" and "Key Mechanisms" (tiling into
 *    on-chip memory, one fused kernel, online softmax, exact result, causal
 *    masking built in), and
 *  - the yelogs.com Flash Attention2-in-Triton article, sections
 *    "核心 Kernel 實現" (per query tile: loop over key/value tiles, running max m,
 *    normaliser l and output accumulator in fp32, final O /= l and stored
 *    statistic m + log l), "因果掩碼的高效實現" (a key is visible iff its position
 *    is <= the query position; key tiles wholly in the future are skipped),
 *    "Softmax 的在線計算" (the rescaling recurrence) and "多查詢注意力（MQA）"
 *    (several query heads sharing one kv head).
 * The statistic is stored with eps = 0, as the natural-log logsumexp of the
 * scaled scores (the article's epilogue adds an eps inside the log; the
 * normaliser is always >= 1, so eps <= 1e-6 moves it by at most 1e-6).
 *
 * Precision. bf16 path: q, k, v, o in bfloat16; both products on bf16 MFMA
 * with fp32 accumulation; scale applied to the fp32 scores (q is never
 * rescaled in bf16); softmax weights rounded to bf16 (nearest even) only as
 * the operand of P.V, while the normaliser sums the fp32 weights; o rounded to
 * nearest even. fp16 path: the same with IEEE half in place of bfloat16.
 * fp32 path: everything in fp32 (fp32 MFMA), no down-conversion.
 *
 * Range. Inputs must be finite (NaN or Inf in q, k or v propagates). Every
 * visible score must satisfy |scale * q.k| < 1.4e9 (|score * log2 e| < 2^31):
 * the weights are exp2(fma(s, c, -m)) with c = |scale| log2 e and m the
 * rounded running max of s*c, so all weights of a row share the factor
 * 2^(m_exact - m), which cancels in O and L but overflows exp2 once the
 * rounding error of m (half an ulp of s*c) exceeds 64. The raw products q.k
 * are also accumulated in fp32, so max|q| * max|k| * D must stay below 3.4e38.
 * Within the range any finite score is handled; the running max starts below
 * every finite fp32 value. L is returned in fp32, so for |L| far above 1 its
 * error is relative (a few ulp of L), not absolute.
 *
 * Layout. Elements are addressed with element strides (batch, token, head);
 * the head-dim stride is 1.
 *   fa_fwd:         q, o contiguous [B, T, H, D]; k, v contiguous [B, T, H_kv, D]
 *   fa_fwd_strided: any non-negative strides (e.g. [B, H, T, D] storage)
 *   lse:            always contiguous float32 [B, H, T]
 *
 * Ownership. All pointers are device memory owned by the caller. The library
 * allocates nothing, frees nothing and keeps no pointer after returning.
 * o and lse must not overlap q, k, v or each other.
 *
 * Execution. Work is enqueued on `stream` (a hipStream_t; NULL = the default
 * stream) and the call returns without synchronising. Inputs must stay valid
 * until that work completes. Calls are thread-safe: the only global state is
 * fa_fwd_splitk_noalloc's scratch (see there).
 *
 * Errors. Arguments are validated completely before any HIP call; on an
 * invalid argument nothing is launched and a nonzero fa_status_t is returned.
 * A launch rejected by the runtime returns FA_ERR_LAUNCH. Faults during
 * execution surface at the caller's next synchronisation, as for any kernel.
 * B == 0 or T == 0 is a valid empty call: it returns FA_OK and launches
 * nothing (pointers may then be NULL).
 */
#ifndef FA_H_
#define FA_H_

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FA_DTYPE_F32 = 0, FA_DTYPE_BF16 = 1, FA_DTYPE_F16 = 2 } fa_dtype_t;

typedef enum {
    FA_OK = 0,
    FA_ERR_NULL_PTR = 1,   /* a required pointer is NULL                       */
    FA_ERR_BAD_SHAPE = 2,  /* B < 0, T < 0, H < 1 or H_kv < 1                  */
    FA_ERR_HEADS = 3,      /* H is not a multiple of H_kv                      */
    FA_ERR_HEAD_DIM = 4,   /* D not in {16, 32, 64, 128}                       */
    FA_ERR_DTYPE = 5,      /* dtype not an fa_dtype_t value                    */
    FA_ERR_SCALE = 6,      /* scale is NaN or infinite                         */
    FA_ERR_ALIGN = 7,      /* q/k/v/o not 16-byte aligned, lse not 4-byte
                              aligned, or a stride not a multiple of 16 bytes  */
    FA_ERR_OVERFLOW = 8,   /* an element offset would exceed 2^62, the grid
                              would exceed 2^24 - 1 work-groups, or T > 2^30   */
    FA_ERR_LAUNCH = 9,     /* the HIP runtime rejected the kernel launch (or,
                              for fa_fwd_splitk_noalloc, the lookup of its
                              scratch address failed)                          */
    FA_ERR_STRIDE = 10,    /* a negative stride                                */
    FA_ERR_WORKSPACE = 11, /* split-K workspace smaller than required          */
    FA_ERR_SCRATCH = 12    /* fa_fwd_splitk_noalloc: the partials would need
                              more than fa_fwd_splitk_scratch_bytes()          */
} fa_status_t;

/*
 * Attention forward on contiguous BNHD tensors.
 *   q    [B, T, H, D]     dtype      read
 *   k, v [B, T, H_kv, D]  dtype      read
 *   o    [B, T, H, D]     dtype      written
 *   lse  [B, H, T]        float32    written (natural-log logsumexp per row)
 *   causal: nonzero = key j visible to query i iff j <= i.
 *   scale:  any finite value, applied to q.k (1/sqrt(D) is the usual choice).
 *   dtype:  FA_DTYPE_BF16, FA_DTYPE_F16 or FA_DTYPE_F32 (applies to q, k, v
 *           and o).
 *   stream: hipStream_t or NULL.
 * Returns an fa_status_t.
 */
int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
           int B, int H, int H_kv, int T, int D, int causal, float scale,
           int dtype, void *stream);

/*
 * Same computation, with element strides {batch, token, head} for each of q,
 * k, v and o (head-dim stride 1). Lets callers pass [B, H, T, D] storage or
 * other views without a copy. Strides must be >= 0 and multiples of 8 (bf16,
 * fp16) or 4 (fp32) elements.
 * Both calls pick the work decomposition from the sizes: the key-range groups
 * of fa_fwd_key_groups below and, with an even number of query heads per kv
 * head and one key-range group (16-bit inputs), work-groups that take the
 * same query tile of two query heads sharing a kv head and stage its K/V
 * tiles once for both; every row's arithmetic, and so the result, is then
 * unchanged bit for bit.
 */
int fa_fwd_strided(const void *q, const void *k, const void *v, void *o, float *lse,
                   int B, int H, int H_kv, int T, int D, int causal, float scale,
                   int dtype, const long long q_strides[3],
                   const long long k_strides[3], const long long v_strides[3],
                   const long long o_strides[3], void *stream);

/*
 * Key-range groups per query tile that fa_fwd and fa_fwd_strided use for these
 * sizes. 2 for bf16/fp16 with D >= 64 when the launch is small: its
 * B * H * ceil(T/128) query tiles are at most a quarter of the 4-wave
 * work-groups the GPU holds at once (1024 at D = 64, 512 at D = 128), or at
 * most all of them with T >= 2048. Otherwise 1. With 2, the work-group of a
 * query tile runs two groups of four waves over the first and the second half
 * of its key tiles and folds the second group's rows into the first's by the
 * online-softmax update of "Softmax 的在線計算" (yelogs.com Flash
 * Attention2-in-Triton article); the result differs from the one-group order
 * only in rounding. Host-only (no HIP call); -1 for invalid sizes or dtype.
 */
int fa_fwd_key_groups(int B, int H, int T, int D, int dtype);

/*
 * Split-K forward (the same result as fa_fwd up to rounding, for bf16 and
 * fp16): the key tiles of every 128-row query tile are divided into nsplit
 * contiguous ranges, each handled by its own work-group, so shapes with few
 * (batch, head) pairs or long causal rows keep the GPU busy. Each range
 * writes a partial result -- attention over its own keys, O_s normalised by
 * its own sum, and L_s = ln of that sum of exp(scores), -inf for an empty
 * range -- and a second kernel merges them:
 *   L = ln sum_s exp(L_s),   O = sum_s exp(L_s - L) O_s,
 * which is the online-softmax update of "Softmax 的在線計算" (yelogs.com Flash
 * Attention2-in-Triton article) applied across ranges instead of tiles.
 * Tensors as in fa_fwd (contiguous BNHD). nsplit >= 1; nsplit == 1 is fa_fwd
 * (workspace unused). workspace: caller-owned device memory, 16-byte
 * aligned, at least fa_fwd_splitk_workspace_bytes(B, H, T, D, nsplit) bytes;
 * its contents are scratch (overwritten; calls sharing one workspace must be
 * ordered on one stream). fp32 inputs return FA_ERR_DTYPE; a workspace too
 * small returns FA_ERR_WORKSPACE. Two kernels are enqueued on `stream`.
 * After the call the workspace holds the partials: float32 O_s
 * [nsplit][B][H][T][D], then float32 L_s [nsplit][B][H][T]. Part s of the
 * 128-row query tile starting at row q0 covers key tiles
 * [s*n/nsplit, (s+1)*n/nsplit) (integer division) of 64 keys each, where
 * n = ceil(kend/64), kend = min(T, q0 + 128) if causal else T.
 */
int fa_fwd_splitk(const void *q, const void *k, const void *v, void *o, float *lse,
                  int B, int H, int H_kv, int T, int D, int causal, float scale,
                  int dtype, int nsplit, void *workspace, long long workspace_bytes,
                  void *stream);

/*
 * fa_fwd_splitk for callers that cannot allocate device memory (code under
 * stream capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same kernels and the same result bit for bit, with the partials kept in a
 * fixed scratch array inside the library instead of a caller workspace. The
 * caller still passes inputs and outputs; nothing is allocated or freed.
 * Limit: the partials, fa_fwd_splitk_workspace_bytes(B, H, T, D, nsplit)
 * bytes, must fit in fa_fwd_splitk_scratch_bytes() (64 MiB), else
 * FA_ERR_SCRATCH and nothing is launched. Every device keeps its own scratch
 * for the life of the process (its address is looked up once per device, on
 * the device of `stream`). All calls on one device share that scratch, which
 * keeps the last call's partials: calls that overlap on one device (e.g. on
 * two streams without ordering) race and give wrong results; order them on
 * one stream. nsplit == 1 uses no scratch (it is fa_fwd).
 */
int fa_fwd_splitk_noalloc(const void *q, const void *k, const void *v, void *o, float *lse,
                          int B, int H, int H_kv, int T, int D, int causal, float scale,
                          int dtype, int nsplit, void *stream);

/* Bytes of the fixed scratch of fa_fwd_splitk_noalloc (64 MiB). */
long long fa_fwd_splitk_scratch_bytes(void);

/*
 * Decode-shaped forward: T_q query rows against a T_k-long key/value cache
 * (bf16 or fp16, contiguous). The query rows are the last T_q positions of the
 * sequence, so query i sits at position T_k - T_q + i and, when causal, sees
 * keys j <= T_k - T_q + i ("因果掩碼的高效實現", yelogs.com Flash
 * Attention2-in-Triton article: key position <= query position); a row that
 * sees no key (T_q > T_k) gets O = 0, L = -inf. This is the inference case
 * "Flash Attention Memory Optimization Explained", "Why It Matters", names
 * (FlashDecoding): few query rows, a long cache. The rows of the H / H_kv
 * query heads sharing a kv head are processed together, so each key/value
 * tile is read once per (batch, kv head, key part), not once per query head;
 * the keys are split into nsplit contiguous ranges of 64-key tiles whose
 * partial results are merged by their logsumexps as in fa_fwd_splitk.
 *   q, o  [B, T_q, H, D]     k, v [B, T_k, H_kv, D]     lse [B, H, T_q] fp32
 *   T_q >= 0 (0: nothing to do), T_k >= 1, nsplit >= 1; workspace: caller's
 *   device memory, 16-byte aligned, at least
 *   fa_fwd_decode_workspace_bytes(B, H, T_q, D, nsplit) bytes (scratch; calls
 *   sharing it must be ordered on one stream). Same range and precision as
 *   fa_fwd_splitk. Two kernels on `stream`. Returns an fa_status_t
 *   (FA_ERR_DTYPE for fp32, FA_ERR_BAD_SHAPE for T_k < 1 or nsplit < 1,
 *   FA_ERR_WORKSPACE for a workspace too small).
 */
int fa_fwd_decode(const void *q, const void *k, const void *v, void *o, float *lse,
                  int B, int H, int H_kv, int T_q, int T_k, int D, int causal, float scale,
                  int dtype, int nsplit, void *workspace, long long workspace_bytes,
                  void *stream);

/* Workspace bytes fa_fwd_decode needs: nsplit * B * H * T_q * (D + 1) * 4;
 * -1 for invalid sizes or overflow. */
long long fa_fwd_decode_workspace_bytes(int B, int H, int T_q, int D, int nsplit);

/*
 * Workspace bytes fa_fwd_splitk needs: nsplit * B * H * T * (D + 1) * 4
 * (fp32 partial outputs, then fp32 partial logsumexps); -1 for invalid sizes
 * or overflow.
 */
long long fa_fwd_splitk_workspace_bytes(int B, int H, int T, int D, int nsplit);

/*
 * Merge n partial results over disjoint key ranges (the combine step of
 * fa_fwd_splitk, exposed for callers that split keys across devices):
 *   o_parts   float32 [n][B][H][T][D]  read  (16-byte aligned)
 *   lse_parts float32 [n][B][H][T]     read  (-inf marks an empty part)
 *   o         [B, T, H, D] contiguous, dtype (bf16, fp16 or fp32), written
 *   lse       float32 [B, H, T], written
 * with L = ln sum_s exp(L_s) and O = sum_s exp(L_s - L) O_s per row; rows
 * whose parts are all empty get O = 0, L = -inf.
 */
int fa_lse_combine(const float *o_parts, const float *lse_parts, int n, int B, int H,
                   int T, int D, void *o, float *lse, int dtype, void *stream);

/*
 * Sparse-pattern forward (bf16 or fp16): the same computation with key j
 * visible to query i iff
 *   |i - j| <= window  or  j is one of the global tokens,
 * and j <= i when causal -- the sliding-window and local-global masks of the
 * yelogs.com Flash Attention2-in-Triton article (sparse-attention variants;
 * the causal flag is applied on top). Key tiles that meet neither the band of
 * a query tile nor a global token are skipped (never loaded).
 *   window        >= 0 (FA_ERR_BAD_SHAPE otherwise); window >= T - 1 with no
 *                 global tokens is fa_fwd.
 *   global_bits   device bitmap of the global tokens as built by
 *                 fa_window_bitmap for this T (bit j%64 of 64-bit word j/64
 *                 set iff key j is global), 8-byte aligned; NULL = none. It
 *                 is read only, so one bitmap serves every call (layer, head
 *                 group, batch) with the same global tokens.
 * Every row sees at least itself, so L is finite. Tensors, dtype (bf16 or
 * fp16; fp32 returns FA_ERR_DTYPE), errors and precision as fa_fwd.
 */
int fa_fwd_window(const void *q, const void *k, const void *v, void *o, float *lse,
                  int B, int H, int H_kv, int T, int D, int causal, float scale,
                  int dtype, int window, const void *global_bits, void *stream);

/*
 * Build the global-token bitmap of fa_fwd_window: global_tokens is a device
 * int32 array of n_global key positions (any order, duplicates allowed;
 * positions outside [0, T) are ignored; NULL allowed when n_global == 0);
 * bits is device memory of at least fa_window_bitmap_bytes(T) bytes, 8-byte
 * aligned, fully overwritten. One kernel on `stream`. FA_ERR_WORKSPACE if
 * bits_bytes is too small.
 */
int fa_window_bitmap(const int *global_tokens, int n_global, int T, void *bits,
                     long long bits_bytes, void *stream);

/* Bytes of the bitmap: 8 * ceil(T / 64); -1 for T < 0. */
long long fa_window_bitmap_bytes(int T);

/*
 * Attention backward: the gradients of the forward above for an upstream
 * gradient dO = dLoss/dO (the loss is taken not to depend on lse). The
 * forward's intermediates are recomputed from q, k and the stored lse instead
 * of being read back ("Flash Attention Memory Optimization Explained", "Key
 * Mechanisms": backward checkpointing); the formulas are the chain rule of the
 * definition above:
 *   P_ij  = exp(s_ij - lse_i) on visible keys, 0 elsewhere
 *   dV_j  = sum_i P_ij dO_i             dP_ij = dO_i . v_j
 *   dS_ij = P_ij (dP_ij - Delta_i),     Delta_i = dO_i . o_i
 *   dQ_i  = scale sum_j dS_ij k_j       dK_j = scale sum_i dS_ij q_i
 * with dK, dV of a kv head summed over the query heads sharing it (in a fixed
 * order: the result is deterministic). Delta uses the identity
 * sum_j P_ij dP_ij = dO_i . o_i, so o and lse must be the forward's outputs
 * for the same q, k, v, causal and scale.
 *   q, o, dout, dq  [B, T, H, D]      dtype (bf16 or fp16), dq written
 *   k, v, dk, dv    [B, T, H_kv, D]   dtype, dk and dv written
 *   lse             [B, H, T]         float32 (the forward's)
 * All contiguous, 16-byte aligned (lse 4-byte). Precision: P and dS are
 * rounded to the input type only as MFMA operands, everything else is fp32;
 * the outputs are rounded to nearest even. fp32 inputs return FA_ERR_DTYPE.
 * head_split: the dK/dV kernel works per (128-key tile, kv head), walking
 * the list of (query head, query tile) pairs that see the tile, heads outer;
 * it can split that list into head_split contiguous parts (whole query heads
 * when head_split divides H / H_kv) whose fp32 sums a reduce kernel adds in
 * a fixed order (still deterministic). A value > 0 is capped at H / H_kv.
 * 0 lets the library choose: enough parts to occupy the GPU, up to H / H_kv,
 * or, with H == H_kv, T >= 4096 and at most 128 (batch, kv head, 128-key
 * tile) work-groups, up to 8 parts of each key tile's query tiles; at D = 128
 * without a window, no more parts than keep the dK/dV launch within 512
 * work-groups when the key tiles alone fit in 512. 1 means no split; < 0 is
 * FA_ERR_BAD_SHAPE.
 * workspace: caller-owned device memory, 16-byte aligned, at least
 * fa_bwd_workspace_bytes(B, H, H_kv, T, D, head_split) bytes: float32 -Delta
 * [B][H][T], float32 lse * log2(e) [B][H][T] (padded to 16 bytes), then with
 * dK/dV parts the fp32 dK and dV parts, then with dQ parts the fp32 dQ parts;
 * overwritten (calls sharing a workspace must be ordered on one stream);
 * FA_ERR_WORKSPACE if too small. dq, dk, dv must not overlap any input, the
 * workspace or each other. Two kernels are enqueued on `stream`, plus one
 * reduce kernel for the dK/dV parts and one for the dQ parts when there are
 * any. On small grids -- at D = 128 the sizes where fa_fwd_key_groups reports
 * 2, at D = 64 at most 192 query tiles of 128 rows, or 384 with T >= 2048 --
 * the dQ kernel splits each query tile's key tiles between two wave groups and
 * adds their fp32 sums; with T >= 4096 and at most 128 query tiles it also
 * splits them into floor(256 / query tiles) parts (at most 8), each a
 * work-group whose fp32 sums the dQ reduce kernel adds in part order. dQ then
 * differs from the one-group order only in rounding.
 */
int fa_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
           const void *dout, void *dq, void *dk, void *dv, int B, int H, int H_kv, int T,
           int D, int causal, float scale, int dtype, int head_split, void *workspace,
           long long workspace_bytes, void *stream);

/*
 * Backward of fa_fwd_window: the gradients above with P restricted to the
 * sliding-window / local-global visible set (|i - j| <= window or j global,
 * and j <= i when causal). o and lse must come from fa_fwd_window with the
 * same window, global_bits, causal and scale. Key tiles that no query sees
 * (outside every band and holding no global token) are skipped on both
 * sides. window >= 0 (FA_ERR_BAD_SHAPE otherwise); global_bits as in
 * fa_fwd_window (NULL = none); everything else as fa_bwd.
 * Workspace: at least fa_bwd_workspace_bytes(...). A tile of 128 keys that
 * holds a global token is seen by queries far outside its band; bytes past
 * that size (fa_bwd_window_workspace_bytes sizes them for n_global tokens)
 * hold per-global-key fp32 partial sums, so that the far queries of such
 * tiles are shared out over several work-groups and added in a fixed order
 * by one more kernel (deterministic). Without them the result is the same
 * up to rounding order, but each such tile is walked by one work-group.
 */
int fa_bwd_window(const void *q, const void *k, const void *v, const void *o,
                  const float *lse, const void *dout, void *dq, void *dk, void *dv, int B,
                  int H, int H_kv, int T, int D, int causal, float scale, int dtype, int window,
                  const void *global_bits, int head_split, void *workspace,
                  long long workspace_bytes, void *stream);

/* Workspace bytes fa_bwd needs for these sizes and head_split (0 = the
 * library's choice, as in fa_bwd): 8 * B * H * T rounded up to 16, plus
 * 8 * parts * B * T * H_kv * D when the dK/dV work is split into parts > 1,
 * plus 4 * dq_parts * B * T * H * D when dQ's keys are split into parts > 1
 * (as described at fa_bwd); -1 for invalid sizes or overflow. */
long long fa_bwd_workspace_bytes(int B, int H, int H_kv, int T, int D, int head_split);

/* Workspace bytes fa_bwd_window needs to split the far queries of up to
 * n_global global tokens (the count the bitmap was built from): the
 * fa_bwd_workspace_bytes size plus, for n_global > 0, a 16-byte header, a
 * slot map (4 bytes a slot, padded to 16) and 8 * slots * parts * B * H_kv * D
 * bytes of fp32 sums, slots = min(n_global, T); parts depends on T, window,
 * the group size and head_split. -1 for invalid sizes (window < 0,
 * n_global < 0) or overflow. After a call, the header's first int32 is the
 * number of global keys whose far queries were split (those of the first 64
 * key tiles holding a global token, as long as all their keys have slots). */
long long fa_bwd_window_workspace_bytes(int B, int H, int H_kv, int T, int D, int window,
                                        int n_global, int head_split);

/* Static, NUL-terminated description of a status code (never NULL). */
const char *fa_status_str(int status);

/* Library version: major * 10000 + minor * 100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
