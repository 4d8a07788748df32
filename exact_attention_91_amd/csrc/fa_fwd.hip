// fa_fwd.hip -- exact, IO-aware, tiled attention forward for MI355X (gfx950):
// the plain forward (fa_fwd, fa_fwd_strided, and fa_fwd_key_groups, which
// reports the kernel variant they pick), its key-split form with the
// logsumexp combine (fa_fwd_splitk, fa_lse_combine), the sliding-window /
// local-global forward and its token bitmap (fa_fwd_window, fa_window_bitmap),
// and their C ABI (include/fa.h).
//
// Method (pages by title and section):
//  * "Flash Attention Memory Optimization Explained" (lzwjava.github.io),
//    "What is Flash Attention?" / "Key Mechanisms": tile Q, K, V into on-chip
//    memory, fuse scale, mask, softmax and the weighted sum into one kernel,
//    normalise rows incrementally with an online softmax; the result is exact.
//  * yelogs.com Flash Attention2-in-Triton article, "核心 Kernel 實現": one
//    program per (batch*head, query tile); fp32 running max m, normaliser l and
//    output accumulator; loop over key/value tiles; epilogue O /= l and the
//    stored statistic m + log l. "因果掩碼的高效實現": key visible iff key
//    position <= query position; the loop stops at the last key tile that
//    touches the query tile. "Softmax 的在線計算": m_new = max(m_old, max s),
//    l_new = exp(m_old - m_new) l_old + sum exp(s - m_new).
//    "多查詢注意力（MQA）": query heads share a kv head (read in place, never
//    expanded).
//
// gfx950 design (not the pages' Triton/CUDA design):
//  * One work-group = 4 waves (256 lanes) = one 128-row query tile of one
//    (batch, head). Each wave owns 32 query rows for the whole key loop.
//  * Scores are computed transposed, S^T = K Q^T, on 32x32 MFMA. In the 32x32
//    accumulator layout lane (col, half) holds column col = query row and 16
//    key rows, so every softmax statistic of a query row lives in one lane pair
//    (lane, lane^32): row max/sum are in-lane reductions plus one
//    v_permlane32_swap, and the rescale factor is a per-lane scalar.
//  * The output is accumulated transposed too, O^T += V^T P^T: P^T is used as
//    the B operand straight from the score registers (no LDS round trip). In
//    the bf16 kernel V stays row-major in LDS and the V^T operand comes from
//    transposing LDS reads (ds_read_b64_tr_b16); the fp32 kernel reads V^T
//    element-wise from a padded row-major tile.
//  * K/V tiles (64 keys, bf16; 32 keys, fp32) are double-buffered in LDS with
//    the next tile's global loads issued before the current tile's math; one
//    barrier per tile. The bf16 kernel copies tiles straight from global
//    memory into LDS (buffer loads to LDS) with XOR-permuted 16-byte chunks;
//    the fp32 kernel stages through registers into padded rows. Either way
//    the MFMA operand reads are bank-conflict free.
//  * The plain, window and two-group forwards (one head per work-group,
//    unsplit) move q and O through LDS (the head-pair kernel O only): the work-group's 128 q rows arrive with the
//    first K/V tile as whole-row buffer loads into the idle second buffer and
//    are read out as MFMA operands; each wave writes its O rows into the
//    buffer the last tile did not use and stores them as whole rows, 16 bytes
//    per lane, instead of 8-byte pieces of 32 rows per instruction. Both the q
//    loads and the O stores carry the non-temporal cache policy (read or
//    written once), which leaves L2 to the K/V tiles that are re-read.
//  * The scale is applied to fp32 scores (folded with log2 e into one FMA
//    before exp2); q is never rescaled in its input precision. A negative scale
//    flips q's sign bits in registers (exact) so the kernel always sees c > 0.
//  * Causal: key tiles past the query tile are never loaded; a wave skips the
//    math of tiles wholly in its future; only tiles that touch the diagonal or
//    the ragged end T are masked element-wise. Query tiles are issued
//    heaviest-first; when the whole grid is resident at once, each round of
//    256 work-groups (one per CU) alternates direction, so a CU's heavy tile
//    of one round is paired with a light one of the next.
//  * Small grids (few query tiles per CU, or long rows with every work-group
//    resident): the G2 instantiation runs 8 waves per work-group in two groups
//    of 4 that take the first and second half of the query tile's key tiles,
//    each with its own LDS buffers, and merges the second group's partial rows
//    into the first's through LDS with the same online-softmax update. Twice
//    the waves per query tile, so MFMA and softmax work of different waves
//    overlap where one wave per SIMD would run them back to back.
//  * Shared kv heads (an even number of query heads per kv head, one key
//    group): the HP instantiation runs 8 waves per work-group, the same query
//    tile of two query heads, which read one set of staged K/V tiles (half
//    the staging and L2 reads per score; per-row arithmetic unchanged).
//  * Variants of the same 16-bit kernel (template flags): SPLIT runs a range
//    of each query tile's key tiles and writes an fp32 partial result that
//    fa_lse_combine_kernel merges by the logsumexps (the online-softmax update
//    of "Softmax 的在線計算" applied across ranges); WINDOW visits only the key
//    tiles that meet the query tile's band or hold a global token (the
//    sparse-attention variants of the same article) and masks by band, token
//    bitmap and causality; DECODE (a SPLIT form) packs the few query rows of
//    the heads that share a kv head into one row tile and copies its K/V tiles,
//    which no other work-group reads, with the non-temporal cache policy.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "fa.h"
#include "fa_device.h"

// Scratch of fa_fwd_splitk_noalloc: the key-split partials live in this
// fixed device array instead of a caller workspace. Every device the library
// runs on holds its own copy for the life of the process; host code reaches it
// only through the per-device address from hipGetSymbolAddress.
constexpr long long kScratchBytes = 64LL << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kBQ = 128;        // query rows per work-group (32 per wave)
constexpr int kCUs = 256;       // MI355X compute units
// Starting value of the running max: below every finite fp32 score, so only
// rows with no visible key (all scores -inf) keep it. exp2(kMaxFloor - m) is 0
// for any finite m above it, and exp2(-inf - kMaxFloor) is 0 for masked keys,
// with no -inf - (-inf) anywhere.
constexpr float kMaxFloor = -3.40282347e38f;

struct FwdParams {
    const void *q, *k, *v;
    void *o;
    float *lse;
    long long qs[3], ks[3], vs[3], os[3];  // element strides {batch, token, head}
    int B, H, H_kv, T;
    int group;      // H / H_kv
    int nq;         // query tiles per (batch, head)
    int nbh;        // B * H
    float c;        // |scale| * log2(e), > 0
    unsigned qsign; // XOR mask applied to q's bits (sign flip for scale < 0)
    // Key-split mode: work-group id = (unit, split s); split s of a query tile
    // covers key tiles [s*n/nsplit, (s+1)*n/nsplit) of its n, and writes its
    // partial result, normalised over its own keys, to opart[s][b][h][t][:]
    // (fp32) and its logsumexp to lpart[s][b][h][t].
    int nsplit;
    float *opart, *lpart;
    // Sliding-window / local-global mode: key j visible to query i iff
    // |i - j| <= window (window clamped to T) or bit j%64 of gbits[j/64] is
    // set (gbits NULL: no global tokens); causal still applies.
    int window;
    const unsigned long long *gbits;
    // 2: two 4-wave groups per work-group split each query tile's key tiles
    // (the G2 kernel); 1: one group.
    int groups;
    // 1: one 8-wave work-group per (query tile, pair of query heads sharing a
    // kv head), the two heads' groups reading one set of staged K/V tiles (the
    // HP kernel); 0: one head per work-group.
    int hpair;
    // Decode mode (the DECODE kernel): Tq query rows, the last Tq positions of
    // the T-long key sequence (query i sits at position T - Tq + i). The rows
    // of the group query heads sharing kv head g are packed, r = hh * Tq + i
    // (head h = g * group + hh), R = group * Tq of them per (batch, kv head);
    // nq counts 128-row tiles of those packed rows.
    int Tq, R;
    // Work-group order: the first `snake` rounds of kCUs work-groups are
    // resident from the start, the i-th work-group of every round on the same
    // CU; odd rounds take their units in reverse, so the CU that starts the
    // heaviest query tile of round 0 gets the lightest one of round 1
    // (0: heaviest first throughout).
    int snake;
};

template <bool B>
struct BoolC {
    static constexpr bool value = B;
};

// Work unit of this work-group: heaviest query tiles first (causal), then
// (batch, head).
struct Unit {
    int b, h, g, q0, s;
};
__device__ __forceinline__ int snake_id(const FwdParams &p) {
    const int id = blockIdx.x;
    const int k = id / kCUs;
    return k < p.snake && (k & 1) ? k * kCUs + kCUs - 1 - (id - k * kCUs) : id;
}

__device__ __forceinline__ Unit unit_of(const FwdParams &p) {
    int id = snake_id(p);
    Unit u;
    u.s = 0;
    if (p.nsplit > 1) {
        u.s = id % p.nsplit;
        id /= p.nsplit;
    }
    const int t = id / p.nbh;
    const int bh = id - t * p.nbh;
    u.b = bh / p.H;
    u.h = bh - u.b * p.H;
    u.g = u.h / p.group;
    u.q0 = (p.nq - 1 - t) * kBQ;
    return u;
}

// ---------------------------------------------------------------------------
// 16-bit kernel (bfloat16 or IEEE half operands, fp32 accumulation), 64-key
// tiles. K and V tiles (two buffers alternating between key tiles) use the
// layout of fa_device.h: K is read as rows (kswz), V transposed for the V^T
// operand of P.V (vswz).
// ---------------------------------------------------------------------------
template <typename E, int D, bool CAUSAL, bool SPLIT, bool WINDOW, bool G2, bool HP = false,
          bool DECODE = false>
__global__ __launch_bounds__(G2 || HP ? 2 * kThreads : kThreads) void fa_fwd_half_kernel(FwdParams p) {
    using L = Bf16Layout<D>;
    using H16 = Half16<E>;
    typedef typename H16::v8 e8_t;
    typedef typename H16::v4 e4_t;
    constexpr int BK = L::BK;
    constexpr int KS = D / 16;              // MFMA k-steps over the head dim
    constexpr int ND = (D + 31) / 32;       // 32-row blocks of O^T
    constexpr int NV = D >= 32 ? D / 32 : 1;  // V^T address variants (one per block)

    static_assert(!G2 || (!SPLIT && !WINDOW && D >= 32), "G2: plain forward, D >= 32");
    static_assert(!HP || (!G2 && !SPLIT && !WINDOW), "HP: plain forward");
    static_assert(!DECODE || (SPLIT && !G2 && !HP && !WINDOW), "DECODE: key-split partials");
    // Two K/V buffers as four distinct LDS variables: the accesses of each loop
    // step name their buffers statically, so the compiler knows the copies into
    // one buffer never alias the operand reads of the other and does not make
    // the reads wait for the copies. With G2 each variable holds both groups'
    // buffers, group g at offset g * TILEB.
    constexpr int NG = G2 ? 2 : 1;
    __shared__ __attribute__((aligned(1024))) unsigned char k_lds0_[NG * L::TILEB];
    __shared__ __attribute__((aligned(1024))) unsigned char v_lds0_[NG * L::TILEB];
    __shared__ __attribute__((aligned(1024))) unsigned char k_lds1_[NG * L::TILEB];
    __shared__ __attribute__((aligned(1024))) unsigned char v_lds1_[NG * L::TILEB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave8 = __builtin_amdgcn_readfirstlane(tid >> 6);
    // G2: key-range group; HP: query head of the pair
    const int grp = G2 || HP ? (wave8 >> 2) : 0;
    const int wave = G2 || HP ? (wave8 & 3) : wave8;   // wave within the group
    // Staging: HP's two groups share one set of K/V buffers and split its loads
    // eight ways; otherwise each group's 4 waves fill their own.
    constexpr int NW = HP ? 8 : 4;
    const int swave = HP ? wave8 : wave;
    unsigned char *const k_lds0 = k_lds0_ + (G2 ? grp : 0) * L::TILEB;
    unsigned char *const v_lds0 = v_lds0_ + (G2 ? grp : 0) * L::TILEB;
    unsigned char *const k_lds1 = k_lds1_ + (G2 ? grp : 0) * L::TILEB;
    unsigned char *const v_lds1 = v_lds1_ + (G2 ? grp : 0) * L::TILEB;
    const int col = lane & 31, half = lane >> 5;
    const int T = p.T;
    Unit u;
    if (HP) {
        // work-group = (query tile, batch, head pair); group g takes head 2 pair + g
        // (both heads read the same kv head: the group size is even)
        const int npair = p.H / 2;
        const int nbp = p.B * npair;
        const int id = snake_id(p);
        const int t = id / nbp;
        const int bp = id - t * nbp;
        u.b = bp / npair;
        u.h = 2 * (bp - u.b * npair) + grp;
        u.g = u.h / p.group;
        u.q0 = (p.nq - 1 - t) * kBQ;
        u.s = 0;
    } else if (DECODE) {
        // work-group = (packed row tile, batch, kv head, split)
        int id = blockIdx.x;
        u.s = id % p.nsplit;
        id /= p.nsplit;
        const int nbg = p.B * p.H_kv;
        const int t = id / nbg;
        const int bg = id - t * nbg;
        u.b = bg / p.H_kv;
        u.g = bg - u.b * p.H_kv;
        u.h = u.g * p.group;
        u.q0 = t * kBQ;
    } else {
        u = unit_of(p);
    }
    const int wq0 = u.q0 + wave * 32;       // first query row of this wave
    const int qrow = wq0 + col;             // this lane's query row (decode: packed row)
    // Decode: this lane's query head and position among the Tq rows, and the
    // last key position its row sees under the causal mask.
    int dh = u.h, di = qrow, dlast = qrow;
    if (DECODE) {
        const int hh = qrow / p.Tq;
        di = qrow - hh * p.Tq;
        dh = u.g * p.group + hh;
        dlast = T - p.Tq + di;
    }
    const bool row_live = DECODE ? qrow < p.R : qrow < T;

    const unsigned short *kbase =
        (const unsigned short *)p.k + u.b * p.ks[0] + u.g * p.ks[2];
    const unsigned short *vbase =
        (const unsigned short *)p.v + u.b * p.vs[0] + u.g * p.vs[2];
    const long long ks1 = p.ks[1], vs1 = p.vs[1];

    // Q fragment = B operand of S^T = K Q^T: lane (col, half) holds
    // q[qrow, 16*ks + 8*half + 0..7].
    // QO (every variant but head pairs and decode, whose q rows are not one
    // head's consecutive rows): the work-group's q rows arrive with the first
    // K/V tile as whole-row buffer loads into the second K/V buffer pair (G2:
    // group 0's, read by both groups) and are read from there as MFMA operands.
    // The others load their q fragments straight into registers. (Every
    // variant writes its output rows through LDS; see the epilogue.)
    constexpr bool QO = !HP && !DECODE;
    e8_t qf[KS];
    if (!QO) {
        const unsigned short *qr = (const unsigned short *)p.q + u.b * p.qs[0] +
                                   dh * p.qs[2] + (long long)di * p.qs[1] + 8 * half;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4_t x = {0u, 0u, 0u, 0u};
            if (row_live) x = *(const u32x4_t *)(qr + 16 * ks);
            x ^= p.qsign;
            qf[ks] = __builtin_bit_cast(e8_t, x);
        }
    }

    // Decode reads every K/V tile once (no other work-group shares it): its
    // copies carry the non-temporal policy. Elsewhere the query tiles of a
    // head re-read each tile and keep the default policy.
    constexpr int KV_POL = DECODE ? kCachePolicyNT : 0;
    const int kend = CAUSAL && !DECODE ? min(T, u.q0 + kBQ) : T;
    const int nkt = (kend + BK - 1) / BK;
    // Key tiles of this work-group: all of them, or split u.s's share; with G2,
    // group 0 takes the first ghalf of them and group 1 the rest.
    const int ghalf = (nkt + 1) / 2;
    const int jbeg = SPLIT ? u.s * nkt / p.nsplit : (G2 && grp ? ghalf : 0);
    const int jend = SPLIT ? (u.s + 1) * nkt / p.nsplit : (G2 && !grp ? ghalf : nkt);
    // Window mode: the key tiles visited are those meeting the band
    // [q0 - window, q_last + window] of this query tile (tiles blo..bhi) and
    // those holding a global token; all others are never loaded.
    int blo = 0, bhi = nkt - 1;
    if (WINDOW) {
        const long long q1 = min(u.q0 + kBQ, T) - 1;
        blo = (int)(max(0LL, (long long)u.q0 - p.window) / BK);
        bhi = (int)(min((long long)kend - 1, q1 + p.window) / BK);
    }
    // The next key tile after j this work-group visits (jend if none).
    auto next_tile = [&](int j) __attribute__((always_inline)) -> int {
        int t = j + 1;
        if (!WINDOW) return t;
        const unsigned long long *gbits = p.gbits;
        if (t < blo) return gbits ? first_nonzero_word(gbits, t, blo) : blo;
        if (t <= bhi) return t;
        return gbits ? first_nonzero_word(gbits, t, jend) : max(t, jend);
    };
    // Global-token bits of tile t, read between steps (never after a step's
    // prefetch is issued, whose loads a wait for this read would include).
    auto tile_bits = [&](int t) __attribute__((always_inline)) -> unsigned long long {
        return (WINDOW && p.gbits && t < jend) ? p.gbits[t] : 0ull;
    };

    // Staging: this wave issues 1 KB loads swave, swave + NW, ... of each tile.
    // Lane slot (row, physical chunk) -> global byte offset within the tile.
    int koff[(L::NLOAD + NW - 1) / NW], voff[(L::NLOAD + NW - 1) / NW];
#pragma unroll
    for (int i = 0; i < (L::NLOAD + NW - 1) / NW; ++i) {
        const int idx = swave + NW * i;
        const int row = idx * L::ROWS_PER_LOAD + lane / L::C;
        const int pc = lane % L::C;
        koff[i] = row * (int)ks1 * 2 + 16 * (pc ^ L::kswz(row));
        voff[i] = row * (int)vs1 * 2 + 16 * (pc ^ L::vswz(row));
    }

    // Loop-invariant LDS byte offsets of this lane's operand reads.
    int kaddr[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        kaddr[ks] = col * L::ROWB + 16 * ((2 * ks + half) ^ L::kswz(col));
    int vaddr[NV];
    {
        const int r0 = 4 * half + ((lane & 15) >> 2);     // row within a 16-key step
        const int dl = (D >= 32 ? 16 * ((lane >> 4) & 1) : 0) + 4 * (lane & 3);
#pragma unroll
        for (int n = 0; n < NV; ++n) {
            const int d = 32 * n + dl;
            vaddr[n] = r0 * L::ROWB + 16 * ((d >> 3) ^ L::vswz(r0)) + 2 * (d & 7);
        }
    }
    const bool vzero = D < 32 && col >= D;  // D=16: rows 16..31 of V^T are zero

    f32x16_t oacc[ND];
#pragma unroll
    for (int n = 0; n < ND; ++n) oacc[n] = f32x16_t{};
    // Running row max in the log2 domain (score * c); kMaxFloor stands for
    // "no visible key yet" (fully masked keys give exp2(-inf) = 0 against it).
    float mref = kMaxFloor;
    float lsum = 0.f;        // this lane's partial normaliser (its 16-key half)
    // The scale lives in a VGPR: a VOP3 FMA with an SGPR operand issues more
    // slowly than one with three VGPR operands.
    float c;
    asm volatile("v_mov_b32 %0, %1" : "=v"(c) : "s"(p.c));
    const bool wave_live = DECODE ? wq0 < p.R : wq0 < T;

    auto tile = [&](bool need_mask, int j, const unsigned char *kt, const unsigned char *vt,
                    unsigned long long gb) {
        const int key0 = j * BK;

        // S^T tile: 64 keys x 32 queries as two 32x32 blocks.
        f32x16_t s0 = f32x16_t{}, s1 = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const e8_t a0 = __builtin_bit_cast(e8_t, *(const lds_bf16x8_t *)(kt + kaddr[ks]));
            const e8_t a1 =
                __builtin_bit_cast(e8_t, *(const lds_bf16x8_t *)(kt + kaddr[ks] + 32 * L::ROWB));
            s0 = H16::mfma(a0, qf[ks], s0);
            s1 = H16::mfma(a1, qf[ks], s1);
        }

        // Element r of block kb is key key0 + 32kb + 8(r/4) + 4half + r%4.
        if (need_mask) {
            const int lim = (CAUSAL ? min(dlast, T - 1) : T - 1) - key0 - 4 * half;
            if (WINDOW) {
                // in the band: lo <= off <= hi; global: bit (off + 4half) of gb
                const int lo = qrow - p.window - key0 - 4 * half;
                const int hi = qrow + p.window - key0 - 4 * half;
                const unsigned long long gl = gb >> (4 * half);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int off = 8 * (r >> 2) + (r & 3);
                    const bool v0 = off <= lim && ((off >= lo && off <= hi) || ((gl >> off) & 1ull));
                    const bool v1 = off + 32 <= lim &&
                                    ((off + 32 >= lo && off + 32 <= hi) || ((gl >> (off + 32)) & 1ull));
                    s0[r] = v0 ? s0[r] : -INFINITY;
                    s1[r] = v1 ? s1[r] : -INFINITY;
                }
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int off = 8 * (r >> 2) + (r & 3);
                    s0[r] = off <= lim ? s0[r] : -INFINITY;
                    s1[r] = off + 32 <= lim ? s1[r] : -INFINITY;
                }
            }
        }

        // Row max over this lane's 32 scores as a chain of 3-input maxima.
        float mx = fmaxf(fmaxf(s0[0], s1[0]), s0[1]);
        mx = fmaxf(mx, s1[1]);
#pragma unroll
        for (int r = 2; r < 16; ++r) mx = fmaxf(fmaxf(mx, s0[r]), s1[r]);
        mx = half_swap_max(mx);
        const float mt = mx * c;
        // Fold the tile into the running max: rows whose max grew rescale
        // their normaliser and output by exp2(m_old - m_new); the others are
        // left alone (the branch is skipped when no row of the wave grew), so
        // each row depends on its own scores alone. The reference stays the
        // exact running max, so the largest weight of a row is exactly 1 and
        // is not rounded when the weights go to bf16. mref starts at a finite
        // floor, so the first visible tile gets alpha = 0 without -inf
        // arithmetic.
        const float mnew = fmaxf(mref, mt);
        if (mnew > mref) {
            const float alpha = fast_exp2(mref - mnew);
            lsum *= alpha;
#pragma unroll
            for (int n = 0; n < ND; ++n) oacc[n] *= alpha;
        }
        mref = mnew;
        const float mr = mref;

        // (the sums start from the first weights: adding them to 0.f would cost
        // two instructions the compiler may not drop, -0.f + 0.f being +0.f)
        s0[0] = fast_exp2(fmaf(s0[0], c, -mr));
        s1[0] = fast_exp2(fmaf(s1[0], c, -mr));
        float ps0 = s0[0], ps1 = s1[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) {
            s0[r] = fast_exp2(fmaf(s0[r], c, -mr));
            s1[r] = fast_exp2(fmaf(s1[r], c, -mr));
            ps0 += s0[r];
            ps1 += s1[r];
        }
        lsum += ps0 + ps1;

        // P^T as the B operand: k-step s4 covers keys 16*s4 .. 16*s4+15; lane
        // half y, element e is key 16*s4 + 8*(e/4) + 4*y + e%4 = register
        // 8*(s4%2) + e of block s4/2.
        e8_t pb[4];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            pb[0][e] = (E)s0[e];
            pb[1][e] = (E)s0[8 + e];
            pb[2][e] = (E)s1[e];
            pb[3][e] = (E)s1[8 + e];
        }
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
#pragma unroll
            for (int n = 0; n < ND; ++n) {
                const unsigned char *va = vt + vaddr[D >= 32 ? n : 0] + 16 * s4 * L::ROWB;
                const e4_t lo = H16::read_tr(va);
                const e4_t hi = H16::read_tr(va + 8 * L::ROWB);
                e8_t a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                if (vzero) a = e8_t{};
                oacc[n] = H16::mfma(a, pb[s4], oacc[n]);
            }
        }
    };

    // One barrier per tile: after it, tile j is in LDS for every wave and every
    // wave has finished reading the buffer that tile j+1 is loaded into. The
    // loop is unrolled by two so each step names its buffers statically.
    auto step = [&](int j, unsigned long long gb, int jn, const unsigned char *kt,
                    const unsigned char *vt, unsigned char *kn, unsigned char *vn) {
        __builtin_amdgcn_s_waitcnt(0);   // this lane's loads of tile j have landed
        __syncthreads();
        // (debug builds: the buffers about to be refilled read as NaN until then;
        // with G2 each group fills its own)
        lds_poison2(jn < jend, kn, vn, L::TILEB, G2 ? (tid & (kThreads - 1)) : tid,
                    HP ? 2 * kThreads : kThreads);
        if (jn < jend)
            stage_tile<D, NW, 64, KV_POL>(kbase, vbase, ks1, vs1, T, jn * BK,
                                           swave, koff, voff, kn, vn);
        const int key0 = j * BK;
        // (decode: every row sees keys up to at least T - Tq, and some row up to T - 1)
        bool active = wave_live && (!CAUSAL || DECODE || key0 <= wq0 + 31) && (!G2 || j < jend);
        bool need_mask = (key0 + BK > T) || (CAUSAL && key0 + BK - 1 > (DECODE ? T - p.Tq : wq0));
        if (WINDOW) {
            // the band of this wave's 32 rows: [wq0 - window, wq0 + 31 + window]
            const long long wlo = (long long)wq0 - p.window, whi = (long long)wq0 + 31 + p.window;
            const bool meets = key0 + BK - 1 >= wlo && key0 <= whi;
            // every row of the wave sees every key of the tile
            const bool inside = key0 >= (long long)wq0 + 31 - p.window &&
                                key0 + BK - 1 <= (long long)wq0 + p.window;
            active = active && (meets || gb != 0ull);
            need_mask = need_mask || !inside;
        }
        if (active) tile(need_mask, j, kt, vt, gb);
    };
    // QO: issue the copies of the work-group's q rows into the second buffer
    // pair (rows q0..q0+63 in k_lds1, q0+64..q0+127 in v_lds1, K tile layout;
    // rows past T arrive as zeros) ...
    auto qo_stage = [&]() __attribute__((always_inline)) {
        if (G2 && grp != 0) return;
        const unsigned short *qb = (const unsigned short *)p.q + u.b * p.qs[0] + u.h * p.qs[2];
        const long long qs1 = p.qs[1];
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
            const int r0 = u.q0 + 64 * hb;
            if (r0 < T)
                stage_rows<D, NW>(qb + (long long)r0 * qs1, qs1, min(T - r0, 64), swave,
                                  hb ? v_lds1_ : k_lds1_);
        }
    };
    // ... and, after the first K/V tile's copies were issued too, wait for all
    // of them: every wave's q rows have landed after the barrier. The first
    // step's wait and barrier then order these reads before the next K/V tile
    // is copied over them.
    auto qo_read = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        const unsigned char *qt = (wave < 2 ? k_lds1_ : v_lds1_) + (wave & 1) * 32 * L::ROWB;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4_t x = __builtin_bit_cast(u32x4_t, *(const lds_bf16x8_t *)(qt + kaddr[ks]));
            x ^= p.qsign;
            qf[ks] = __builtin_bit_cast(e8_t, x);
        }
    };
    // Buffer pair (0 or 1) of the last step: the other one is free at the end.
    bool last0 = true;
    if (WINDOW) {
        int j = next_tile(-1);
        unsigned long long gj = tile_bits(j);
        if (QO) qo_stage();
        if (j < jend)
            stage_tile<D, NW, 64, KV_POL>(kbase, vbase, ks1, vs1, T, j * BK,
                                           swave, koff, voff, k_lds0, v_lds0);
        if (QO) qo_read();
        while (j < jend) {
            const int jn = next_tile(j);
            const unsigned long long gn = tile_bits(jn);
            step(j, gj, jn, k_lds0, v_lds0, k_lds1, v_lds1);
            last0 = true;
            if (jn >= jend) break;
            const int jnn = next_tile(jn);
            const unsigned long long gnn = tile_bits(jnn);
            step(jn, gn, jnn, k_lds1, v_lds1, k_lds0, v_lds0);
            last0 = false;
            j = jnn;
            gj = gnn;
        }
    } else if (G2) {
        // Both groups take ghalf steps, one barrier each; group 1's last step is
        // idle when nkt is odd (no staging, no math).
        if (QO) qo_stage();
        if (jbeg < jend)
            stage_tile<D, NW, 64, KV_POL>(kbase, vbase, ks1, vs1, T, jbeg * BK,
                                           swave, koff, voff, k_lds0, v_lds0);
        if (QO) qo_read();
        for (int i = 0; i < ghalf; i += 2) {
            step(jbeg + i, 0ull, jbeg + i + 1, k_lds0, v_lds0, k_lds1, v_lds1);
            if (i + 1 < ghalf)
                step(jbeg + i + 1, 0ull, jbeg + i + 2, k_lds1, v_lds1, k_lds0, v_lds0);
        }
    } else {
        if (QO) qo_stage();
        if (jbeg < jend)
            stage_tile<D, NW, 64, KV_POL>(kbase, vbase, ks1, vs1, T, jbeg * BK,
                                           swave, koff, voff, k_lds0, v_lds0);
        if (QO) qo_read();
        last0 = ((jend - 1 - jbeg) & 1) == 0;
        for (int j = jbeg; j < jend; j += 2) {
            step(j, 0ull, j + 1, k_lds0, v_lds0, k_lds1, v_lds1);
            if (j + 1 < jend) step(j + 1, 0ull, j + 2, k_lds1, v_lds1, k_lds0, v_lds0);
        }
    }

    if (G2) {
        // Merge: wave w + 4 (group 1) leaves its O^T accumulators, running max and
        // row sum in LDS, lane-major; wave w (group 0, the same 32 rows) folds them
        // in with the online-softmax update m = max(m0, m1), x = x0 2^(m0 - m) +
        // x1 2^(m1 - m). A group that saw no key of a row holds the floor max and
        // zero sums, so its factor is 0. Every wave takes both barriers; after the
        // first, all K/V reads are done and the buffers are free.
        static_assert(!G2 || (ND * 16 + 2) * 64 * 4 <= NG * L::TILEB, "merge area");
        __syncthreads();
        float *mb = (float *)(wave == 0 ? k_lds0_ : wave == 1 ? v_lds0_
                              : wave == 2 ? k_lds1_ : v_lds1_);
        const float lrow = half_swap_sum(lsum);
        if (grp == 1 && wave_live) {
#pragma unroll
            for (int n = 0; n < ND; ++n)
#pragma unroll
                for (int r = 0; r < 16; ++r) mb[(n * 16 + r) * 64 + lane] = oacc[n][r];
            mb[ND * 16 * 64 + lane] = mref;
            mb[(ND * 16 + 1) * 64 + lane] = lrow;
        }
        __syncthreads();
        if (grp == 1) return;
        if (wave_live) {
            const float m1 = mb[ND * 16 * 64 + lane];
            const float l1 = mb[(ND * 16 + 1) * 64 + lane];
            const float m = fmaxf(mref, m1);
            const float a0 = fast_exp2(mref - m), a1 = fast_exp2(m1 - m);
#pragma unroll
            for (int n = 0; n < ND; ++n)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    oacc[n][r] = oacc[n][r] * a0 + mb[(n * 16 + r) * 64 + lane] * a1;
            // the merged row sum, held by the half-0 lane (the epilogue adds halves)
            lsum = half ? 0.f : lrow * a0 + l1 * a1;
            mref = m;
        }
    }

    // HP and the key split: every wave has finished reading the K/V tiles
    // before any wave reuses their buffers for its output rows.
    if (HP || (SPLIT && !DECODE)) __syncthreads();
    if (!wave_live) return;
    const float lt = half_swap_sum(lsum);
    if (DECODE && !row_live) return;   // (others: every lane takes part in the LDS transposes)
    const float inv = lt > 0.f ? __builtin_amdgcn_rcpf(lt) : 0.f;
    const float lse_row = lt > 0.f ? (mref + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
    if (DECODE) {
        // Partial result over this split's keys, normalised by its own l, fp32,
        // stored from registers: a decode step writes few rows, which do not pay
        // for the barrier and the transpose.
        float *orow = p.opart + ((((long long)u.s * p.B + u.b) * p.H + dh) * p.Tq + di) * D;
#pragma unroll
        for (int n = 0; n < ND; ++n)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int d = 32 * n + 8 * rg + 4 * half;
                if (D >= 32 || d < D) {
                    f32x4_t o4;
#pragma unroll
                    for (int e = 0; e < 4; ++e) o4[e] = oacc[n][4 * rg + e] * inv;
                    *(f32x4_t *)(orow + d) = o4;
                }
            }
        if (half == 0) p.lpart[(((long long)u.s * p.B + u.b) * p.H + dh) * p.Tq + di] = lse_row;
        return;
    }
    // O^T register r of block n is dim 32n + 8(r/4) + 4half + r%4 of this lane's
    // row (col). The rows go out through LDS: each wave writes its 32 rows into
    // a region of its own, 16-byte chunk c of a row at c XOR a function of the
    // row, and reads them back a row-contiguous 16 bytes per lane, so the global
    // stores cover whole rows (non-temporal: written once).
    if (SPLIT) {
        // Partial result over this split's keys, normalised by its own l, fp32:
        // 32 rows x 4D bytes = one K/V buffer per wave (all free after the
        // barrier above); a wave's rows are consecutive query rows.
        constexpr int C = D / 4;                   // 16-byte chunks of an fp32 row
        constexpr int RB = 4 * D;                  // bytes of an fp32 row
        static_assert(32 * RB <= L::TILEB, "fp32 rows of a wave fit one buffer");
        unsigned char *ob = wave == 0 ? k_lds0 : wave == 1 ? v_lds0 : wave == 2 ? k_lds1 : v_lds1;
#ifdef FA_LDS_POISON
        for (int i = lane; i < 2 * RB; i += 64)    // 32 rows: NaN until written
            *(lds_u32x4_t *)(ob + 16 * i) = u32x4_t{~0u, ~0u, ~0u, ~0u};
#endif
#pragma unroll
        for (int n = 0; n < ND; ++n)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int d = 32 * n + 8 * rg + 4 * half;
                if (D >= 32 || d < D) {
                    f32x4_t o4;
#pragma unroll
                    for (int e = 0; e < 4; ++e) o4[e] = oacc[n][4 * rg + e] * inv;
                    *(lds_f32x4_t *)(ob + col * RB + 16 * ((d >> 2) ^ (col & (C - 1)))) = o4;
                }
            }
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_wave_barrier();
        // partial row index of the wave's row r (-1: past T)
        auto prow = [&](int r) -> long long {
            const int pr = wq0 + r;
            return pr < T ? (((long long)u.s * p.B + u.b) * p.H + u.h) * T + pr : -1;
        };
#pragma unroll
        for (int i = 0; i < C / 2; ++i) {
            const int r = i * (64 / C) + lane / C;
            const int c = lane % C;
            const f32x4_t x = *(const lds_f32x4_t *)(ob + r * RB + 16 * (c ^ (r & (C - 1))));
            const long long row = prow(r);
            if (row >= 0) __builtin_nontemporal_store(x, (f32x4_t *)(p.opart + row * D + 4 * c));
        }
        if (half == 0 && row_live) p.lpart[prow(col)] = lse_row;
        return;
    }
    // QO: the buffer pair that did not hold the last tile is free: its last reads
    // (the tile before) and copies ended before the last step's barrier (with
    // no step at all it still holds q, each wave's rows where that wave's O rows
    // go, read by the wave itself before it writes there). HP: wave8 takes half
    // of buffer wave8 / 2 (all four are free after the barrier above). G2:
    // group-0 wave w's merge area (it has read its partner's values).
    constexpr int C = L::C;
    auto oswz = [](int r) { return (r >> 1) & (C - 1); };
    const int hb = wave8 >> 1;
    unsigned char *ob =
        HP   ? (hb == 0 ? k_lds0 : hb == 1 ? v_lds0 : hb == 2 ? k_lds1 : v_lds1) +
                   (wave8 & 1) * 32 * L::ROWB
        : G2 ? (wave == 0 ? k_lds0_ : wave == 1 ? v_lds0_ : wave == 2 ? k_lds1_ : v_lds1_)
             : (last0 ? (wave < 2 ? k_lds1 : v_lds1) : (wave < 2 ? k_lds0 : v_lds0)) +
                   (wave & 1) * 32 * L::ROWB;
#ifdef FA_LDS_POISON
    for (int i = lane; i < 2 * L::ROWB; i += 64)   // 32 rows: NaN until written
        *(lds_u32x4_t *)(ob + 16 * i) = u32x4_t{~0u, ~0u, ~0u, ~0u};
#endif
#pragma unroll
    for (int n = 0; n < ND; ++n)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            const int d = 32 * n + 8 * rg + 4 * half;
            if (D >= 32 || d < D) {
                e4_t o4;
#pragma unroll
                for (int e = 0; e < 4; ++e) o4[e] = (E)(oacc[n][4 * rg + e] * inv);
                *(lds_u32x2_t *)(ob + col * L::ROWB + 16 * ((d >> 3) ^ oswz(col)) + 8 * half) =
                    __builtin_bit_cast(u32x2_t, o4);
            }
        }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    unsigned short *obase = (unsigned short *)p.o + u.b * p.os[0] + u.h * p.os[2];
#pragma unroll
    for (int i = 0; i < C / 2; ++i) {
        const int r = i * (64 / C) + lane / C;
        const int c = lane % C;
        const u32x4_t x = *(const lds_u32x4_t *)(ob + r * L::ROWB + 16 * (c ^ oswz(r)));
        if (wq0 + r < T)
            __builtin_nontemporal_store(x,
                                        (u32x4_t *)(obase + (long long)(wq0 + r) * p.os[1] + 8 * c));
    }
    if (half == 0 && row_live) p.lse[((long long)u.b * p.H + u.h) * T + qrow] = lse_row;
}
// ---------------------------------------------------------------------------
// fp32 kernel: fp32 operands on fp32 MFMA (32x32x2), 32-key tiles. Weights stay
// fp32 for P.V.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void fa_fwd_f32_kernel(FwdParams p) {
    constexpr int BK = 32;
    constexpr int KS = D / 2;               // MFMA k-steps over the head dim
    constexpr int ND = (D + 31) / 32;
    constexpr int KST = D + 1;              // odd stride: column reads hit 32 banks
    constexpr int VST = D;
    constexpr int CH = BK * D / 4;          // float4 chunks per tile
    constexpr int CPT = (CH + kThreads - 1) / kThreads;

    __shared__ __attribute__((aligned(16))) float k_lds[2][BK * KST];
    __shared__ __attribute__((aligned(16))) float v_lds[2][BK * VST];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int col = lane & 31, half = lane >> 5;
    const int T = p.T;
    const Unit u = unit_of(p);
    const int wq0 = u.q0 + wave * 32;
    const int qrow = wq0 + col;

    const float *kbase = (const float *)p.k + u.b * p.ks[0] + u.g * p.ks[2];
    const float *vbase = (const float *)p.v + u.b * p.vs[0] + u.g * p.vs[2];

    // Q fragment: lane (col, half) holds q[qrow, 2*ks + half].
    float qf[KS];
    {
        const float *qr = (const float *)p.q + u.b * p.qs[0] + u.h * p.qs[2] +
                          (long long)qrow * p.qs[1];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            unsigned x = 0u;
            if (qrow < T) x = __float_as_uint(qr[2 * ks + half]);
            qf[ks] = __uint_as_float(x ^ p.qsign);
        }
    }

    const int kend = CAUSAL ? min(T, u.q0 + kBQ) : T;
    const int nkt = (kend + BK - 1) / BK;

    f32x4_t kreg[CPT], vreg[CPT];
    auto load_tile = [&](int j) {
        const int key0 = j * BK;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = tid + i * kThreads;
            if (CH % kThreads == 0 || c < CH) {
                const int row = c / (D / 4), dc = c % (D / 4);
                const int key = key0 + row;
                f32x4_t x = {0.f, 0.f, 0.f, 0.f}, y = {0.f, 0.f, 0.f, 0.f};
                if (key < T) {
                    x = *(const f32x4_t *)(kbase + (long long)key * p.ks[1] + 4 * dc);
                    y = *(const f32x4_t *)(vbase + (long long)key * p.vs[1] + 4 * dc);
                }
                kreg[i] = x;
                vreg[i] = y;
            }
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = tid + i * kThreads;
            if (CH % kThreads == 0 || c < CH) {
                const int row = c / (D / 4), dc = c % (D / 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) k_lds[buf][row * KST + 4 * dc + e] = kreg[i][e];
                *(f32x4_t *)&v_lds[buf][row * VST + 4 * dc] = vreg[i];
            }
        }
    };

    f32x16_t oacc[ND];
#pragma unroll
    for (int n = 0; n < ND; ++n) oacc[n] = f32x16_t{};
    float mc = -INFINITY, lsum = 0.f;
    // The scale lives in a VGPR: a VOP3 FMA with an SGPR operand issues more
    // slowly than one with three VGPR operands.
    float c;
    asm volatile("v_mov_b32 %0, %1" : "=v"(c) : "s"(p.c));
    const bool wave_live = wq0 < T;

    load_tile(0);
    for (int j = 0; j < nkt; ++j) {
        const int buf = j & 1;
        // (debug builds: buffer buf, last read at step j - 2, reads as NaN until
        // its refill)
        lds_poison(true, k_lds[buf], sizeof(k_lds[0]), tid, kThreads);
        lds_poison(true, v_lds[buf], sizeof(v_lds[0]), tid, kThreads);
        store_tile(buf);
        __syncthreads();
        if (j + 1 < nkt) load_tile(j + 1);

        const int key0 = j * BK;
        const bool active = wave_live && (!CAUSAL || key0 <= wq0 + 31);
        if (!active) continue;

        // S^T block: 32 keys x 32 queries; register r is key key0 + 8(r/4) + 4half + r%4.
        f32x16_t s = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            s = __builtin_amdgcn_mfma_f32_32x32x2f32(k_lds[buf][col * KST + 2 * ks + half],
                                                     qf[ks], s, 0, 0, 0);

        const bool need_mask = (key0 + BK > T) || (CAUSAL && key0 + BK - 1 > wq0);
        if (need_mask) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = key0 + 8 * (r >> 2) + 4 * half + (r & 3);
                const bool vis = key < T && (!CAUSAL || key <= qrow);
                s[r] = vis ? s[r] : -INFINITY;
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
        mx = half_swap_max(mx);
        const float mc_new = fmaxf(mc, mx * c);
        const float mref = (mc_new == -INFINITY) ? 0.f : mc_new;
        const float alpha = fast_exp2(mc - mref);
        mc = mc_new;
        float psum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            s[r] = fast_exp2(fmaf(s[r], c, -mref));
            psum += s[r];
        }
        lsum = fmaf(lsum, alpha, psum);
#pragma unroll
        for (int n = 0; n < ND; ++n) oacc[n] *= alpha;

        // O^T += V^T P^T, k-step st: lane half y supplies key 8(st/4) + 4y + st%4,
        // which is its own score register st.
#pragma unroll
        for (int n = 0; n < ND; ++n)
#pragma unroll
            for (int st = 0; st < 16; ++st) {
                const int key = 8 * (st >> 2) + 4 * half + (st & 3);
                float a = 0.f;
                if (D >= 32 || col < D) a = v_lds[buf][key * VST + 32 * n + col];
                oacc[n] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, s[st], oacc[n], 0, 0, 0);
            }
    }

    if (!wave_live) return;
    const float lt = half_swap_sum(lsum);
    if (qrow >= T) return;
    const float inv = lt > 0.f ? __builtin_amdgcn_rcpf(lt) : 0.f;
    float *orow = (float *)p.o + u.b * p.os[0] + (long long)qrow * p.os[1] + u.h * p.os[2];
#pragma unroll
    for (int n = 0; n < ND; ++n)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            const int d = 32 * n + 8 * rg + 4 * half;
            if (D >= 32 || d < D) {
                f32x4_t o4;
#pragma unroll
                for (int e = 0; e < 4; ++e) o4[e] = oacc[n][4 * rg + e] * inv;
                *(f32x4_t *)(orow + d) = o4;
            }
        }
    if (half == 0)
        p.lse[((long long)u.b * p.H + u.h) * T + qrow] =
            lt > 0.f ? (mc + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// Combine of partial results over disjoint key ranges. For every row,
//   L = ln sum_s e^{L_s},  O = sum_s e^{L_s - L} O_s,
// the same merge the online softmax applies between two key tiles ("Softmax
// 的在線計算": rescale each partial by exp(m_s - m_new)). Rows with no key
// in any part (all L_s = -inf) get O = 0 and L = -inf. Each thread handles
// four consecutive dims of one row; parts are fp32 [n][B][H][T][D] and
// [n][B][H][T]; o is written in its own dtype with element strides os.
// ---------------------------------------------------------------------------
struct CombineParams {
    const float *opart, *lpart;
    void *o;
    float *lse;
    long long os[3];
    int n, B, H, T;
};

template <typename E, int D>
__global__ __launch_bounds__(256) void fa_lse_combine_kernel(CombineParams p) {
    constexpr int TPR = D / 4;                  // threads per row
    const long long rows = (long long)p.B * p.H * p.T;
    const long long row = (long long)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
    const int d = 4 * (threadIdx.x % TPR);
    if (row >= rows) return;
    // One pass, merging part by part with a running max (the online-softmax
    // update): every load is independent of the arithmetic, so the loads of
    // an unrolled group are all in flight together. Each partial is read once
    // (non-temporal loads).
    const float *lp = p.lpart + row;
    const float *op = p.opart + row * D + d;
    float m = -INFINITY, l = 0.f;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    auto merge = [&](float ls, f32x4_t os) __attribute__((always_inline)) {
        if (ls > -INFINITY) {
            const float mn = fmaxf(m, ls);
            const float a = expf(m - mn), w = expf(ls - mn);
            l = fmaf(l, a, w);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = fmaf(acc[e], a, w * os[e]);
            m = mn;
        }
    };
    int s = 0;
    for (; s + 4 <= p.n; s += 4) {
        float ls[4];
        f32x4_t os[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ls[i] = lp[(s + i) * rows];
            os[i] = __builtin_nontemporal_load((const f32x4_t *)(op + (s + i) * rows * D));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) merge(ls[i], os[i]);
    }
    for (; s < p.n; ++s)
        merge(lp[s * rows], __builtin_nontemporal_load((const f32x4_t *)(op + s * rows * D)));
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const float L = l > 0.f ? m + logf(l) : -INFINITY;
    const int t = (int)(row % p.T);
    const long long bh = row / p.T;
    const int h = (int)(bh % p.H), b = (int)(bh / p.H);
    E *orow = (E *)p.o + b * p.os[0] + (long long)t * p.os[1] + h * p.os[2] + d;
    typedef E e4v __attribute__((ext_vector_type(4)));
    e4v o4;
#pragma unroll
    for (int e = 0; e < 4; ++e) o4[e] = (E)(acc[e] * inv);
    *(e4v *)orow = o4;
    if (d == 0) p.lse[row] = L;
}

// ---------------------------------------------------------------------------
// Per-key-tile bitmaps of the global tokens: word w has bit t set iff key
// 64w + t is in the list. One thread per word scans the list, staged through
// LDS 256 positions at a time (one coalesced load per chunk), so no zeroing
// pass or atomics are needed; positions outside [0, T) match no word.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void fa_global_bits_kernel(const int *idx, int n, int T,
                                                             unsigned long long *bits,
                                                             int nwords) {
    __shared__ int chunk[256];
    const int w = blockIdx.x * 256 + threadIdx.x;
    unsigned long long word = 0ull;
    for (int base = 0; base < n; base += 256) {
        const int m = min(256, n - base);
        __syncthreads();                  // the previous chunk has been read
        if ((int)threadIdx.x < m) chunk[threadIdx.x] = idx[base + threadIdx.x];
        __syncthreads();
        for (int i = 0; i < m; ++i) {
            const int j = chunk[i];
            if (j >= 0 && j < T && (j >> 6) == w) word |= 1ull << (j & 63);
        }
    }
    if (w < nwords) bits[w] = word;
}

// ---------------------------------------------------------------------------
// Host side: validation (no HIP calls), dispatch, launch.
// ---------------------------------------------------------------------------
constexpr long long kMaxOffset = 1LL << 62;
constexpr int kMaxT = (1 << 30);    // longest sequence accepted (32-bit row arithmetic)
constexpr long long kNumCU = kCUs;
constexpr long long kMaxGrid = (1LL << 24) - 1;

// Largest element offset + 1 of a [B, T, heads, D] view; -1 on overflow.
long long extent(const long long s[3], int B, int T, int heads, int D) {
    long long e = D, t;
    const long long n[3] = {B - 1LL, T - 1LL, heads - 1LL};
    for (int i = 0; i < 3; ++i) {
        if (__builtin_mul_overflow(n[i], s[i], &t) || __builtin_add_overflow(e, t, &e))
            return -1;
    }
    return e;
}

bool aligned(const void *ptr, uintptr_t a) { return ((uintptr_t)ptr % a) == 0; }

// Work-groups of kernel K resident on one CU when it runs alone (asked of the
// runtime once per kernel; 0 if the query fails).
template <void (*K)(FwdParams)>
int resident_per_cu(int threads) {
    static const int n = [threads] {
        int b = 0;
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, (const void *)K, threads, 0) ==
                       hipSuccess
                   ? b
                   : 0;
    }();
    return n;
}

// Launch K with the causal work-group order balanced per CU when the whole
// grid is resident at once (work-groups i, i + kCUs, i + 2 kCUs, ... then all
// run on one CU): its full rounds are snaked. A larger grid keeps the
// heaviest-first order, which the hardware's dynamic dispatch balances;
// uniform (non-causal) work has nothing to balance.
template <void (*K)(FwdParams)>
hipError_t launch_fwd(dim3 grid, dim3 block, hipStream_t stream, FwdParams p, bool causal) {
    if (causal) {
        const long long resident = (long long)kCUs * resident_per_cu<K>((int)block.x);
        p.snake = (long long)grid.x <= resident ? (int)(grid.x / kCUs) : 0;
    }
    return launch_kernel(K, grid, block, stream, p);
}

template <int D, bool CAUSAL, bool SPLIT, bool WINDOW>
hipError_t launch(const FwdParams &p, int dtype, dim3 grid, hipStream_t stream) {
    constexpr bool CAN_G2 = D >= 64 && !SPLIT && !WINDOW;
    constexpr bool CAN_HP = !SPLIT && !WINDOW;
    const dim3 b4(kThreads), b8(2 * kThreads);
    if (CAN_HP && p.hpair && dtype == FA_DTYPE_BF16)
        return launch_fwd<fa_fwd_half_kernel<__bf16, D, CAUSAL, SPLIT, WINDOW, false, CAN_HP>>(
            grid, b8, stream, p, CAUSAL);
    else if (CAN_HP && p.hpair && dtype == FA_DTYPE_F16)
        return launch_fwd<fa_fwd_half_kernel<_Float16, D, CAUSAL, SPLIT, WINDOW, false, CAN_HP>>(
            grid, b8, stream, p, CAUSAL);
    else if (CAN_G2 && p.groups == 2 && dtype == FA_DTYPE_BF16)
        return launch_fwd<fa_fwd_half_kernel<__bf16, D, CAUSAL, SPLIT, WINDOW, CAN_G2>>(
            grid, b8, stream, p, CAUSAL);
    else if (CAN_G2 && p.groups == 2 && dtype == FA_DTYPE_F16)
        return launch_fwd<fa_fwd_half_kernel<_Float16, D, CAUSAL, SPLIT, WINDOW, CAN_G2>>(
            grid, b8, stream, p, CAUSAL);
    else if (dtype == FA_DTYPE_BF16)
        return launch_fwd<fa_fwd_half_kernel<__bf16, D, CAUSAL, SPLIT, WINDOW, false>>(
            grid, b4, stream, p, CAUSAL);
    else if (dtype == FA_DTYPE_F16)
        return launch_fwd<fa_fwd_half_kernel<_Float16, D, CAUSAL, SPLIT, WINDOW, false>>(
            grid, b4, stream, p, CAUSAL);
    else if (!SPLIT && !WINDOW)
        return launch_fwd<fa_fwd_f32_kernel<D, CAUSAL>>(grid, b4, stream, p, CAUSAL);
    return hipErrorInvalidValue;   // callers validate dtype first; not reached
}

// The decode kernel: packed query rows of the heads sharing a kv head, key
// split into parts whose partials fa_lse_combine_kernel merges.
template <int D, bool CAUSAL>
hipError_t launch_decode(const FwdParams &p, int dtype, dim3 grid, hipStream_t stream) {
    if (dtype == FA_DTYPE_BF16)
        return launch_kernel(
            (fa_fwd_half_kernel<__bf16, D, CAUSAL, true, false, false, false, true>), grid,
            dim3(kThreads), stream, p);
    return launch_kernel(
        (fa_fwd_half_kernel<_Float16, D, CAUSAL, true, false, false, false, true>), grid,
        dim3(kThreads), stream, p);
}

template <bool CAUSAL, bool SPLIT, bool WINDOW = false>
int launch_d(const FwdParams &p, int D, int dtype, dim3 grid, hipStream_t stream) {
    hipError_t e;
    switch (D) {
        case 16: e = launch<16, CAUSAL, SPLIT, WINDOW>(p, dtype, grid, stream); break;
        case 32: e = launch<32, CAUSAL, SPLIT, WINDOW>(p, dtype, grid, stream); break;
        case 64: e = launch<64, CAUSAL, SPLIT, WINDOW>(p, dtype, grid, stream); break;
        default: e = launch<128, CAUSAL, SPLIT, WINDOW>(p, dtype, grid, stream); break;
    }
    return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// Validation shared by the entry points (no HIP calls) and the kernel
// parameters. Sets *empty for B == 0 or T == 0 (a valid no-op).
int prepare(const void *q, const void *k, const void *v, const void *o, const float *lse,
            int B, int H, int H_kv, int T, int D, float scale, int dtype,
            const long long q_strides[3], const long long k_strides[3],
            const long long v_strides[3], const long long o_strides[3], FwdParams *pp,
            bool *empty) {
    *empty = false;
    if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16)
        return FA_ERR_DTYPE;
    const bool half16 = dtype != FA_DTYPE_F32;   // a 16-bit element type
    if (B < 0 || T < 0 || H < 1 || H_kv < 1) return FA_ERR_BAD_SHAPE;
    if (H % H_kv != 0) return FA_ERR_HEADS;
    if (D != 16 && D != 32 && D != 64 && D != 128) return FA_ERR_HEAD_DIM;
    if (!isfinite(scale)) return FA_ERR_SCALE;
    float c = fabsf(scale) * kLog2e;
    if (!isfinite(c)) return FA_ERR_SCALE;
    if (B == 0 || T == 0) {
        *empty = true;
        return FA_OK;
    }
    if (!q || !k || !v || !o || !lse || !q_strides || !k_strides || !v_strides || !o_strides)
        return FA_ERR_NULL_PTR;
    const long long *st[4] = {q_strides, k_strides, v_strides, o_strides};
    for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 3; ++j)
            if (st[i][j] < 0) return FA_ERR_STRIDE;
    const long long vec = half16 ? 8 : 4;  // elements per 16 bytes
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
        !aligned(lse, 4))
        return FA_ERR_ALIGN;
    for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 3; ++j)
            if (st[i][j] % vec != 0) return FA_ERR_ALIGN;
    const long long eq = extent(q_strides, B, T, H, D), eo = extent(o_strides, B, T, H, D);
    const long long ek = extent(k_strides, B, T, H_kv, D), ev = extent(v_strides, B, T, H_kv, D);
    if (eq < 0 || eo < 0 || ek < 0 || ev < 0 || eq > kMaxOffset || eo > kMaxOffset ||
        ek > kMaxOffset || ev > kMaxOffset)
        return FA_ERR_OVERFLOW;
    // The 16-bit kernel addresses 64 rows of q, k or v with 32-bit byte offsets.
    if (half16) {
        const long long s1 = std::max(q_strides[1], std::max(k_strides[1], v_strides[1]));
        if (64 * 2 * s1 + 2 * D > (1LL << 31) - 1) return FA_ERR_OVERFLOW;
    }
    // Kernels index rows and round T up to whole tiles in 32-bit ints.
    if (T > kMaxT) return FA_ERR_OVERFLOW;
    const long long nq = ((long long)T + kBQ - 1) / kBQ;
    const long long nbh = (long long)B * H;
    if (nbh > kMaxGrid || nbh * nq > kMaxGrid || nbh * T > kMaxOffset) return FA_ERR_OVERFLOW;

    FwdParams &p = *pp;
    p.q = q; p.k = k; p.v = v; p.o = (void *)o; p.lse = (float *)lse;
    for (int j = 0; j < 3; ++j) {
        p.qs[j] = q_strides[j]; p.ks[j] = k_strides[j];
        p.vs[j] = v_strides[j]; p.os[j] = o_strides[j];
    }
    p.B = B; p.H = H; p.H_kv = H_kv; p.T = T;
    p.group = H / H_kv;
    p.nq = (int)nq;
    p.nbh = (int)nbh;
    // scale == 0 means uniform weights; the smallest normal c reproduces them
    // exactly in fp32 (every c*s rounds to a value whose exp2 is 1).
    p.c = c > 0.f ? c : 1.17549435e-38f;
    p.qsign = scale < 0.f ? (half16 ? 0x80008000u : 0x80000000u) : 0u;
    p.nsplit = 1;
    p.opart = p.lpart = nullptr;
    p.window = 0;
    p.gbits = nullptr;
    p.groups = 1;
    p.hpair = 0;
    p.Tq = T;
    p.R = 0;
    p.snake = 0;
    return FA_OK;
}

void contiguous_strides(int T, int heads, int D, long long s[3]) {
    s[0] = (long long)T * heads * D;
    s[1] = (long long)heads * D;
    s[2] = D;
}

// Bytes of split-K workspace: fp32 partial outputs then partial logsumexps;
// -1 on overflow.
long long splitk_bytes(int B, int H, int T, int D, int nsplit) {
    long long rows, r;
    if (__builtin_mul_overflow((long long)B * H, (long long)T, &rows) ||
        __builtin_mul_overflow(rows, (long long)nsplit, &rows) ||
        __builtin_mul_overflow(rows, (long long)(D + 1) * 4, &r))
        return -1;
    return r;
}

int launch_combine(const float *opart, const float *lpart, int n, int B, int H, int T, int D,
                   void *o, const long long os[3], float *lse, int dtype, hipStream_t stream) {
    CombineParams c;
    c.opart = opart; c.lpart = lpart; c.o = o; c.lse = lse;
    for (int j = 0; j < 3; ++j) c.os[j] = os[j];
    c.n = n; c.B = B; c.H = H; c.T = T;
    const long long rows = (long long)B * H * T;
    const long long per_block = 256 / (D / 4);
    const long long blocks = (rows + per_block - 1) / per_block;
    if (blocks > kMaxGrid) return FA_ERR_OVERFLOW;
    const dim3 grid((unsigned)blocks);
    hipError_t e;
#define FA_COMBINE(E, DD) \
    e = launch_kernel((fa_lse_combine_kernel<E, DD>), grid, dim3(256), stream, c)
#define FA_COMBINE_D(E)                          \
    switch (D) {                                 \
        case 16: FA_COMBINE(E, 16); break;       \
        case 32: FA_COMBINE(E, 32); break;       \
        case 64: FA_COMBINE(E, 64); break;       \
        default: FA_COMBINE(E, 128); break;      \
    }
    if (dtype == FA_DTYPE_BF16) {
        FA_COMBINE_D(__bf16)
    } else if (dtype == FA_DTYPE_F16) {
        FA_COMBINE_D(_Float16)
    } else {
        FA_COMBINE_D(float)
    }
#undef FA_COMBINE_D
#undef FA_COMBINE
    return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// Two key-range groups per query tile (the G2 kernel) when the grid is small:
// at most a quarter of the 4-wave work-group slots (256 CUs x 4, or x 2 at
// D = 128 by registers), or rows of 2048 keys or more with every work-group
// resident at once. Elsewhere the single-group kernel is faster.
int key_groups(long long units, int T, int D, int dtype) {
    const long long slots = kNumCU * (D >= 128 ? 2 : 4);
    return dtype != FA_DTYPE_F32 && D >= 64 &&
                   (units <= slots / 4 || (T >= 2048 && units <= slots))
               ? 2
               : 1;
}

}  // namespace

extern "C" int fa_fwd_key_groups(int B, int H, int T, int D, int dtype) {
    if (B < 0 || H < 1 || T < 0 || (D != 16 && D != 32 && D != 64 && D != 128) ||
        (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16))
        return -1;
    return key_groups(mul_sat(mul_sat(B, H), ((long long)T + kBQ - 1) / kBQ), T, D, dtype);
}

extern "C" int fa_fwd_strided(const void *q, const void *k, const void *v, void *o, float *lse,
                              int B, int H, int H_kv, int T, int D, int causal, float scale,
                              int dtype, const long long q_strides[3],
                              const long long k_strides[3], const long long v_strides[3],
                              const long long o_strides[3], void *stream) {
    FwdParams p;
    bool empty;
    const int st = prepare(q, k, v, o, lse, B, H, H_kv, T, D, scale, dtype, q_strides, k_strides,
                           v_strides, o_strides, &p, &empty);
    if (st != FA_OK || empty) return st;
    const long long units = (long long)p.nbh * p.nq;
    p.groups = key_groups(units, T, D, dtype);
    p.hpair = p.groups == 1 && dtype != FA_DTYPE_F32 && p.group % 2 == 0 ? 1 : 0;
    const dim3 grid((unsigned)(p.hpair ? units / 2 : units));
    hipStream_t s = (hipStream_t)stream;
    return causal ? launch_d<true, false>(p, D, dtype, grid, s)
                  : launch_d<false, false>(p, D, dtype, grid, s);
}

extern "C" int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                      int H, int H_kv, int T, int D, int causal, float scale, int dtype,
                      void *stream) {
    long long qs[3], ks[3];
    contiguous_strides(T, H, D, qs);
    contiguous_strides(T, H_kv, D, ks);
    return fa_fwd_strided(q, k, v, o, lse, B, H, H_kv, T, D, causal, scale, dtype, qs, ks, ks,
                          qs, stream);
}

extern "C" long long fa_fwd_splitk_workspace_bytes(int B, int H, int T, int D, int nsplit) {
    if (B < 0 || H < 1 || T < 0 || nsplit < 1 || (D != 16 && D != 32 && D != 64 && D != 128))
        return -1;
    return splitk_bytes(B, H, T, D, nsplit);
}

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];   // per device: address of `scratch`, once looked up

// Device address of `scratch` on the device that owns `stream` (the current
// device for the NULL stream), looked up with that device current the first
// time and kept.
int scratch_address(hipStream_t stream, void **out) {
    int dev = -1;
    if (stream ? hipStreamGetDevice(stream, &dev) != hipSuccess : hipGetDevice(&dev) != hipSuccess)
        return FA_ERR_LAUNCH;
    if (dev < 0 || dev >= kMaxDevices) return FA_ERR_LAUNCH;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return FA_ERR_LAUNCH;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return FA_ERR_LAUNCH;
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (cur != dev && hipSetDevice(cur) != hipSuccess) return FA_ERR_LAUNCH;
        if (e != hipSuccess || !ptr) return FA_ERR_LAUNCH;
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return FA_OK;
}

// fa_fwd_splitk with its partials in `workspace`, or, when use_scratch is set,
// in the library's fixed scratch (workspace arguments ignored).
int splitk_impl(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                int H_kv, int T, int D, int causal, float scale, int dtype, int nsplit,
                void *workspace, long long workspace_bytes, void *stream, bool use_scratch) {
    long long qs[3], ks[3];
    contiguous_strides(T, H, D, qs);
    contiguous_strides(T, H_kv, D, ks);
    FwdParams p;
    bool empty;
    int st = prepare(q, k, v, o, lse, B, H, H_kv, T, D, scale, dtype, qs, ks, ks, qs, &p, &empty);
    if (st != FA_OK) return st;
    if (nsplit < 1) return FA_ERR_BAD_SHAPE;
    if (dtype == FA_DTYPE_F32) return FA_ERR_DTYPE;   // key split runs on the 16-bit kernel
    if (empty) return FA_OK;
    if (nsplit == 1)
        return fa_fwd_strided(q, k, v, o, lse, B, H, H_kv, T, D, causal, scale, dtype, qs, ks,
                              ks, qs, stream);
    const long long need = splitk_bytes(B, H, T, D, nsplit);
    if (need < 0) return FA_ERR_OVERFLOW;
    const long long units = (long long)p.nbh * p.nq;
    if (units * nsplit > kMaxGrid) return FA_ERR_OVERFLOW;
    hipStream_t s = (hipStream_t)stream;
    if (use_scratch) {
        if (need > kScratchBytes) return FA_ERR_SCRATCH;
        st = scratch_address(s, &workspace);
        if (st != FA_OK) return st;
    } else {
        if (!workspace) return FA_ERR_NULL_PTR;
        if (workspace_bytes < need) return FA_ERR_WORKSPACE;
        if (!aligned(workspace, 16)) return FA_ERR_ALIGN;
    }
    const long long rows = (long long)B * H * T;
    p.nsplit = nsplit;
    p.opart = (float *)workspace;
    p.lpart = p.opart + rows * nsplit * D;
    const dim3 grid((unsigned)(units * nsplit));
    const int ls = causal ? launch_d<true, true>(p, D, dtype, grid, s)
                          : launch_d<false, true>(p, D, dtype, grid, s);
    if (ls != FA_OK) return ls;
    return launch_combine(p.opart, p.lpart, nsplit, B, H, T, D, o, qs, lse, dtype, s);
}

}  // namespace

extern "C" int fa_fwd_splitk(const void *q, const void *k, const void *v, void *o, float *lse,
                             int B, int H, int H_kv, int T, int D, int causal, float scale,
                             int dtype, int nsplit, void *workspace, long long workspace_bytes,
                             void *stream) {
    return splitk_impl(q, k, v, o, lse, B, H, H_kv, T, D, causal, scale, dtype, nsplit,
                       workspace, workspace_bytes, stream, false);
}

extern "C" int fa_fwd_splitk_noalloc(const void *q, const void *k, const void *v, void *o,
                                     float *lse, int B, int H, int H_kv, int T, int D,
                                     int causal, float scale, int dtype, int nsplit,
                                     void *stream) {
    return splitk_impl(q, k, v, o, lse, B, H, H_kv, T, D, causal, scale, dtype, nsplit, nullptr,
                       0, stream, true);
}

extern "C" long long fa_fwd_splitk_scratch_bytes(void) { return kScratchBytes; }

extern "C" long long fa_fwd_decode_workspace_bytes(int B, int H, int Tq, int D, int nsplit) {
    if (B < 0 || H < 1 || Tq < 0 || nsplit < 1 || (D != 16 && D != 32 && D != 64 && D != 128))
        return -1;
    return splitk_bytes(B, H, Tq, D, nsplit);
}

extern "C" int fa_fwd_decode(const void *q, const void *k, const void *v, void *o, float *lse,
                             int B, int H, int H_kv, int Tq, int Tk, int D, int causal,
                             float scale, int dtype, int nsplit, void *workspace,
                             long long workspace_bytes, void *stream) {
    if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16) return FA_ERR_DTYPE;
    if (B < 0 || Tq < 0 || Tk < 1 || H < 1 || H_kv < 1 || nsplit < 1) return FA_ERR_BAD_SHAPE;
    if (H % H_kv != 0) return FA_ERR_HEADS;
    if (D != 16 && D != 32 && D != 64 && D != 128) return FA_ERR_HEAD_DIM;
    if (!isfinite(scale)) return FA_ERR_SCALE;
    const float c = fabsf(scale) * kLog2e;
    if (!isfinite(c)) return FA_ERR_SCALE;
    if (B == 0 || Tq == 0) return FA_OK;
    if (Tq > kMaxT || Tk > kMaxT) return FA_ERR_OVERFLOW;
    if (!q || !k || !v || !o || !lse || !workspace) return FA_ERR_NULL_PTR;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
        !aligned(workspace, 16) || !aligned(lse, 4))
        return FA_ERR_ALIGN;
    long long qs[3], ks[3];
    contiguous_strides(Tq, H, D, qs);
    contiguous_strides(Tk, H_kv, D, ks);
    const long long eq = extent(qs, B, Tq, H, D), ek = extent(ks, B, Tk, H_kv, D);
    if (eq < 0 || ek < 0 || eq > kMaxOffset || ek > kMaxOffset) return FA_ERR_OVERFLOW;
    const long long rows = (long long)(H / H_kv) * Tq;     // packed rows per (batch, kv head)
    if (rows > kMaxT) return FA_ERR_OVERFLOW;
    const long long nq = (rows + kBQ - 1) / kBQ;
    const long long units = mul_sat(mul_sat(B, H_kv), nq);
    if (units > kMaxGrid || units * nsplit > kMaxGrid) return FA_ERR_OVERFLOW;
    const long long need = splitk_bytes(B, H, Tq, D, nsplit);
    if (need < 0) return FA_ERR_OVERFLOW;
    if (workspace_bytes < need) return FA_ERR_WORKSPACE;

    FwdParams p;
    p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
    for (int j = 0; j < 3; ++j) {
        p.qs[j] = qs[j]; p.os[j] = qs[j];
        p.ks[j] = ks[j]; p.vs[j] = ks[j];
    }
    p.B = B; p.H = H; p.H_kv = H_kv; p.T = Tk;
    p.group = H / H_kv;
    p.nq = (int)nq;
    p.nbh = (int)mul_sat(B, H);
    p.c = c > 0.f ? c : 1.17549435e-38f;
    p.qsign = scale < 0.f ? 0x80008000u : 0u;
    p.nsplit = nsplit;
    p.opart = (float *)workspace;
    p.lpart = p.opart + (long long)B * H * Tq * nsplit * D;
    p.window = 0;
    p.gbits = nullptr;
    p.groups = 1;
    p.hpair = 0;
    p.Tq = Tq;
    p.R = (int)rows;
    const dim3 grid((unsigned)(units * nsplit));
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    switch (D) {
        case 16: e = causal ? launch_decode<16, true>(p, dtype, grid, s)
                            : launch_decode<16, false>(p, dtype, grid, s); break;
        case 32: e = causal ? launch_decode<32, true>(p, dtype, grid, s)
                            : launch_decode<32, false>(p, dtype, grid, s); break;
        case 64: e = causal ? launch_decode<64, true>(p, dtype, grid, s)
                            : launch_decode<64, false>(p, dtype, grid, s); break;
        default: e = causal ? launch_decode<128, true>(p, dtype, grid, s)
                            : launch_decode<128, false>(p, dtype, grid, s); break;
    }
    if (e != hipSuccess) return FA_ERR_LAUNCH;
    return launch_combine(p.opart, p.lpart, nsplit, B, H, Tq, D, o, qs, lse, dtype, s);
}

extern "C" int fa_lse_combine(const float *o_parts, const float *lse_parts, int n, int B, int H,
                              int T, int D, void *o, float *lse, int dtype, void *stream) {
    if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16)
        return FA_ERR_DTYPE;
    if (n < 1 || B < 0 || H < 1 || T < 0) return FA_ERR_BAD_SHAPE;
    if (D != 16 && D != 32 && D != 64 && D != 128) return FA_ERR_HEAD_DIM;
    if (B == 0 || T == 0) return FA_OK;
    if (!o_parts || !lse_parts || !o || !lse) return FA_ERR_NULL_PTR;
    if (!aligned(o_parts, 16) || !aligned(lse_parts, 4) || !aligned(o, 16) || !aligned(lse, 4))
        return FA_ERR_ALIGN;
    if (splitk_bytes(B, H, T, D, n) < 0 || (long long)B * H * T * D > kMaxOffset)
        return FA_ERR_OVERFLOW;
    long long os[3];
    contiguous_strides(T, H, D, os);
    return launch_combine(o_parts, lse_parts, n, B, H, T, D, o, os, lse, dtype,
                          (hipStream_t)stream);
}

extern "C" long long fa_window_bitmap_bytes(int T) {
    if (T < 0) return -1;
    return 8LL * ((T + 63LL) / 64);
}

extern "C" int fa_window_bitmap(const int *global_tokens, int n_global, int T, void *bits,
                                long long bits_bytes, void *stream) {
    if (n_global < 0 || T < 0) return FA_ERR_BAD_SHAPE;
    if (T == 0) return FA_OK;
    if (!bits || (n_global > 0 && !global_tokens)) return FA_ERR_NULL_PTR;
    if (!aligned(bits, 8) || !aligned(global_tokens, 4)) return FA_ERR_ALIGN;
    const long long need = fa_window_bitmap_bytes(T);
    if (bits_bytes < need) return FA_ERR_WORKSPACE;
    const int nwords = (int)(need / 8);
    const hipError_t e = launch_kernel(fa_global_bits_kernel, dim3((nwords + 255) / 256),
                                       dim3(256), (hipStream_t)stream, global_tokens, n_global,
                                       T, (unsigned long long *)bits, nwords);
    return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

extern "C" int fa_fwd_window(const void *q, const void *k, const void *v, void *o, float *lse,
                             int B, int H, int H_kv, int T, int D, int causal, float scale,
                             int dtype, int window, const void *global_bits, void *stream) {
    long long qs[3], ks[3];
    contiguous_strides(T, H, D, qs);
    contiguous_strides(T, H_kv, D, ks);
    FwdParams p;
    bool empty;
    const int st = prepare(q, k, v, o, lse, B, H, H_kv, T, D, scale, dtype, qs, ks, ks, qs, &p,
                           &empty);
    if (st != FA_OK) return st;
    if (window < 0) return FA_ERR_BAD_SHAPE;
    if (dtype == FA_DTYPE_F32) return FA_ERR_DTYPE;   // the masks run on the 16-bit kernel
    if (empty) return FA_OK;
    if (!aligned(global_bits, 8)) return FA_ERR_ALIGN;
    p.window = window < T ? window : T;   // a window of T already sees every key
    p.gbits = (const unsigned long long *)global_bits;
    const dim3 grid((unsigned)((long long)p.nbh * p.nq));
    hipStream_t s = (hipStream_t)stream;
    return causal ? launch_d<true, false, true>(p, D, dtype, grid, s)
                  : launch_d<false, false, true>(p, D, dtype, grid, s);
}

extern "C" const char *fa_status_str(int status) {
    switch (status) {
        case FA_OK: return "ok";
        case FA_ERR_NULL_PTR: return "null pointer argument";
        case FA_ERR_BAD_SHAPE: return "bad shape: need B >= 0, T >= 0, H >= 1, H_kv >= 1";
        case FA_ERR_HEADS: return "H must be a multiple of H_kv";
        case FA_ERR_HEAD_DIM: return "head dim D must be 16, 32, 64 or 128";
        case FA_ERR_DTYPE: return "dtype must be FA_DTYPE_F32, FA_DTYPE_BF16 or FA_DTYPE_F16";
        case FA_ERR_SCALE: return "scale must be finite (and |scale|*log2(e) finite)";
        case FA_ERR_ALIGN:
            return "misaligned: q/k/v/o need 16-byte alignment and 16-byte-multiple strides, "
                   "lse 4-byte alignment";
        case FA_ERR_OVERFLOW:
            return "size overflow: offsets beyond 2^62, grid beyond 2^24-1 or T beyond 2^30";
        case FA_ERR_LAUNCH: return "kernel launch failed";
        case FA_ERR_STRIDE: return "negative stride";
        case FA_ERR_WORKSPACE:
            return "workspace smaller than fa_fwd_splitk_workspace_bytes() for these sizes";
        case FA_ERR_SCRATCH:
            return "sizes need more than the library's fixed scratch "
                   "(fa_fwd_splitk_scratch_bytes()); call fa_fwd_splitk with a workspace";
        default: return "unknown status";
    }
}

extern "C" int fa_version(void) { return 100; }
