// fa_bwd.hip -- attention backward for MI355X (gfx950), and its C ABI
// (fa_bwd, fa_bwd_window, fa_bwd_workspace_bytes, fa_bwd_window_workspace_bytes
// in include/fa.h).
//
// Method: "Flash Attention Memory Optimization Explained" (lzwjava.github.io),
// "Key Mechanisms", backward checkpointing -- the backward pass recomputes the
// forward's intermediates (scores, weights) from q, k and the stored
// per-row logsumexp L instead of keeping the T x T matrices. The gradients are
// the chain rule of the forward's definition:
//   P = exp(scale QK^T - L),  dV = P^T dO,  dP = dO V^T,
//   dS = P o (dP - Delta),  Delta_i = dO_i . O_i,  dQ = scale dS K,  dK = scale dS^T Q.
//
// gfx950 design (two kernels on one stream, three with a head split; no
// atomics, deterministic):
//  * fa_bwd_dkdv_kernel: one work-group per 128-key tile of one (batch, kv
//    head); each wave keeps its 32 keys' K and V rows in registers as MFMA
//    operands and its dK, dV accumulators in registers for the whole loop,
//    and streams 64-row tiles of Q, dO (and their L2, -Delta) of every query
//    head of the group through double-buffered LDS. Scores are computed as
//    S = Q K^T, so a lane owns one key column: P and dS feed the B operand of
//    dV^T += dO^T P and dK^T += Q^T dS straight from registers, with dO^T and
//    Q^T read from the same LDS tiles by transposing reads. At D = 128 two
//    variants fit two waves per SIMD: V rows in LDS with 32-row tiles (VL), or
//    K rows in LDS with 8-wave work-groups whose two wave groups share each
//    64-row tile's staging and take one 32-row block each (KL).
//  * fa_bwd_dq_kernel (first): the forward's decomposition (one work-group
//    per 128-row query tile, heaviest causal tiles first); each wave keeps
//    its 32 query rows of Q and dO in registers, forms Delta = rowsum(dO o O)
//    and L2 = L log2(e) for them (-Delta and L2 stored in the workspace for
//    the dK/dV kernel), streams K and V tiles, computes S^T = K Q^T and dP^T = V dO^T,
//    and accumulates dQ^T += K^T dS^T with K^T from transposing reads of the
//    K tile. At D = 64 and 128 on small grids its 8-wave G2 instantiation
//    splits each query tile's key tiles between two groups of 4 waves and adds
//    the second group's dQ^T into the first's through LDS.
//  * fa_bwd_reduce_kernel (dK/dV parts only): adds the fp32 parts in order;
//    fa_bwd_dq_reduce_kernel does the same for dQ key parts (long rows, few
//    query tiles: the two-group dQ kernel's key tiles split over work-groups).
//  * Window mode (fa_bwd_window): both main kernels visit only the tiles that
//    meet a tile's band or hold a global token. A key tile holding a global
//    token is seen by far queries too; with workspace slots for the global
//    keys, those far query tiles are shared out to extra dK/dV work-groups
//    whose fp32 sums fa_bwd_gsum_kernel adds in a fixed order.
//  Tiles read both as rows and transposed use the dual swizzle (dswz) of
//  fa_device.h. Causal: key tiles wholly after a query tile are never loaded;
//  query tiles wholly before a key tile are never loaded; waves skip the math
//  of blocks wholly masked; only blocks that touch the diagonal or the ragged
//  end T are masked element-wise.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fa.h"
#include "fa_device.h"

namespace {

constexpr int kBlk = 128;   // query rows (dQ) or keys (dK/dV) per work-group

struct BwdParams {
    const void *q, *k, *v, *o, *dout;
    const float *lse;
    void *dq, *dk, *dv;
    float *delta, *l2;      // workspace, [B][H][T] each
    int B, H, H_kv, T;
    int group;              // H / H_kv
    int nblk;               // 128-row tiles per sequence
    // 2: the dQ kernel splits each query tile's key tiles between two groups
    // of 4 waves (8-wave work-groups, D >= 64, plain masks); 1: one group.
    int dq_groups;
    // dQ key parts (two-group kernel only): work-group (query tile, part s)
    // takes key tiles [s*n/dq_parts, (s+1)*n/dq_parts) of the tile's n and,
    // with dq_parts > 1, writes fp32 sums (unscaled) to dqpart[s][b][t][h][d];
    // fa_bwd_dq_reduce_kernel adds them in part order.
    int dq_parts;
    float *dqpart;
    float c;                // scale * log2(e) (signed)
    float scale;
    // Split of the dK/dV kernel: work-group (key tile, b, g, part s) takes
    // items [s*n/hsplit, (s+1)*n/hsplit) of the key tile's list of n =
    // group * nper (query head, query tile) items, heads outer -- whole query
    // heads [s*group/hsplit, (s+1)*group/hsplit) when hsplit divides group.
    // With hsplit > 1 each part writes fp32 sums (dK unscaled) to
    // dkpart/dvpart [s][b][t][g][d], added in part order by the reduce kernel.
    int hsplit;
    float *dkpart, *dvpart;
    // 1: the D = 128 dK/dV kernel keeps V rows in LDS and walks 32-row query
    // tiles (two work-groups per CU); 0: V in registers, 64-row tiles.
    int vlds;
    // 1: the D = 128 dK/dV kernel with K rows in LDS and 8-wave work-groups
    int klds;
    // Window mode (as the window forward): key j visible to query i iff
    // |i - j| <= window (clamped to T) or bit j%64 of gbits[j/64] is set
    // (gbits NULL: no global tokens); causal still applies.
    int window;
    const unsigned long long *gbits;
    int nwords;             // 64-bit words of gbits: ceil(T / 64)
    // Window split of the global key tiles (nslots > 0). A key tile holding
    // a global token is seen by every query (causal: every later one), not
    // only by its band. Its main work-group then walks the band alone, like
    // every other tile, and the far query tiles (outside the band: there only
    // the global keys are visible) go to nfar = B * H_kv * nchunk extra
    // work-groups, chunk c taking run c of the (query head, far tile) list.
    // For each global key, every part writes its fp32 sums (dK unscaled) to
    // the key's slot, its rank among the global keys:
    //   gpk / gpv [slot][part][b][g][D],  part = head part hs (band) or
    //   hsplit + c (far chunk c),  nparts = hsplit + nchunk,
    // gmeta[0] = number of slots in use, gmeta[4 + slot] = the slot's key;
    // fa_bwd_gsum_kernel adds the parts in order. Only the first kMaxSplit
    // global tiles whose keys all have slots (rank < nslots) are split; the
    // others keep the full walk.
    int nslots, nchunk, nparts, nfar;
    int *gmeta;
    float *gpk, *gpv;
};

constexpr int kMaxSplit = 64;   // global key tiles that can be split

// Global key tiles in key order, from a scan of the bitmap (two words per
// 128-key tile, bits at or past T ignored) by the whole work-group.
struct SplitLds {
    int tile[kMaxSplit];     // the r-th tile holding a global token
    int before[kMaxSplit];   // global keys in the tiles before it
    int end[kMaxSplit];      // ... and in it
    int wsum[4][2];
    int nelig;               // eligible tiles: a prefix of the list
    int mine;                // rank of tile tk among the global tiles (-1: none)
};

__device__ __forceinline__ unsigned long long gword(const BwdParams &p, int w) {
    if (w >= p.nwords) return 0ull;
    unsigned long long x = p.gbits[w];
    const int tail = p.T - 64 * w;
    if (tail < 64) x &= (1ull << tail) - 1ull;
    return x;
}

// Called by every thread of the work-group (it synchronises).
__device__ void scan_global_tiles(const BwdParams &p, int tk, SplitLds &sl) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) sl.mine = -1;
    int nt = 0, nk = 0;   // global tiles / keys before this chunk (uniform)
    for (int c0 = 0; c0 < p.nblk && nt < kMaxSplit; c0 += kThreads) {
        const int t = c0 + tid;
        unsigned long long w0 = 0ull, w1 = 0ull;
        if (t < p.nblk) {
            w0 = gword(p, 2 * t);
            w1 = gword(p, 2 * t + 1);
        }
        const int f = (w0 | w1) != 0ull;
        const int kc = __popcll(w0) + __popcll(w1);
        int sf = f, sk = kc;   // inclusive scans within the wave
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int xf = __shfl_up(sf, o), xk = __shfl_up(sk, o);
            if (lane >= o) {
                sf += xf;
                sk += xk;
            }
        }
        if (lane == 63) {
            sl.wsum[wave][0] = sf;
            sl.wsum[wave][1] = sk;
        }
        __syncthreads();
        int pf = nt, pk = nk;
        for (int w = 0; w < 4; ++w) {
            if (w < wave) {
                pf += sl.wsum[w][0];
                pk += sl.wsum[w][1];
            }
        }
        for (int w = 0; w < 4; ++w) {
            nt += sl.wsum[w][0];
            nk += sl.wsum[w][1];
        }
        const int rank = pf + sf - f;
        if (f && rank < kMaxSplit) {
            sl.tile[rank] = t;
            sl.before[rank] = pk + sk - kc;
            sl.end[rank] = pk + sk;
        }
        if (f && t == tk) sl.mine = rank;
        __syncthreads();   // wsum is rewritten by the next chunk
    }
    if (tid == 0) {
        const int nl = min(nt, kMaxSplit);
        int n = 0;
        while (n < nl && sl.end[n] <= p.nslots) ++n;
        sl.nelig = n;
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// dK, dV. Work-group: keys [k0, k0 + 128) of kv head g of batch b, wave w
// owns keys wk0 = k0 + 32w .. wk0 + 31 (lane col = key wk0 + col).
// Query tiles: 64 rows; LDS holds Q and dO tiles (dual swizzle) and the
// tile's L2 and -Delta (64 floats each), two buffers alternating.
// In the 32x32 accumulator layout of S = Q K^T (a 32-query block x 32 keys),
// lane (col, half) register r is query 8(r/4) + 4half + r%4 of the block and
// key col: the B operand of the 32-query reduction for k-step s2 is
// registers 8 s2 .. 8 s2 + 7, whose queries 16 s2 + 8(e/4) + 4half + e%4 are
// exactly the rows the transposing reads of dO^T / Q^T hand lane (d, half).
// ---------------------------------------------------------------------------
template <typename E, int D, bool CAUSAL, bool WINDOW, bool VL = false, bool KL = false>
__global__ __launch_bounds__(KL ? 2 * kThreads : kThreads) void fa_bwd_dkdv_kernel(BwdParams p) {
    // VL (D = 128 only): the V rows of the work-group's 128 keys live in LDS
    // (read as MFMA operands) instead of 32 registers per lane, and query tiles
    // are 32 rows, so that the kernel fits 256 registers and two work-groups
    // share a CU (two waves per SIMD). Otherwise V stays in registers and query
    // tiles are 64 rows (D = 128: one work-group per CU).
    // KL (D = 128 only): 8 waves per work-group, the K rows of its 128 keys in
    // LDS (read as MFMA operands, like VL's V rows), V in registers, 64-row
    // query tiles staged once for all 8 waves; waves w and w + 4 own the same 32
    // keys and take the first and second 32-row block of each tile, and wave
    // w + 4 adds its dK/dV sums into wave w's at the end. Two waves per SIMD
    // with 64-row tiles and no spilled registers.
    static_assert(!VL || (D == 128 && !WINDOW), "VL: plain masks, D = 128");
    static_assert(!KL || (D == 128 && !WINDOW && !VL), "KL: plain masks, D = 128");
    constexpr int NW = KL ? 8 : 4;            // waves per work-group
    constexpr int NT = NW * 64;
    using L = Bf16Layout<D, VL ? 32 : 64>;
    using H16 = Half16<E>;
    typedef typename H16::v8 e8_t;
    typedef typename H16::v4 e4_t;
    constexpr int BQ = L::BK;               // query rows per staged tile
    constexpr int NSUB = BQ / 32;           // 32-row blocks per tile
    constexpr int KS = D / 16;              // k-steps over the head dim
    constexpr int ND = (D + 31) / 32;       // 32-row blocks of dK^T / dV^T
    constexpr int NI = (L::NLOAD + NW - 1) / NW;

    __shared__ __attribute__((aligned(1024))) unsigned char q_lds0[L::TILEB];
    __shared__ __attribute__((aligned(1024))) unsigned char o_lds0[L::TILEB];
    __shared__ __attribute__((aligned(1024))) unsigned char q_lds1[L::TILEB];
    __shared__ __attribute__((aligned(1024))) unsigned char o_lds1[L::TILEB];
    __shared__ __attribute__((aligned(16))) float st_lds0[2 * BQ];   // L2 then -Delta
    __shared__ __attribute__((aligned(16))) float st_lds1[2 * BQ];
    __shared__ __attribute__((aligned(1024))) unsigned char v_rows[VL ? kBlk * L::ROWB : 16];
    __shared__ __attribute__((aligned(1024))) unsigned char k_rows[KL ? kBlk * L::ROWB : 16];
    __shared__ SplitLds sl;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave8 = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = KL ? (wave8 >> 2) : 0;       // KL: 32-row block of each query tile
    const int wave = KL ? (wave8 & 3) : wave8;   // 32-key block
    const int swave = KL ? wave8 : wave;          // share of the tile copies
    const int col = lane & 31, half = lane >> 5;
    const int T = p.T;
    const int nbg = p.B * p.H_kv;
    // Work-group: with the window split the first nfar work-groups are far
    // parts (b, g, chunk); the others are (key tile, b, g, head part), key
    // tile 0 (most work) first.
    int blk = blockIdx.x;
    const bool far = WINDOW && blk < p.nfar;
    int hs = 0, chunk = 0, tk0 = 0, bg;
    if (far) {
        chunk = blk % p.nchunk;
        bg = blk / p.nchunk;
    } else {
        if (WINDOW) blk -= p.nfar;
        hs = blk % p.hsplit;
        const int id = blk / p.hsplit;
        tk0 = id / nbg;
        bg = id - tk0 * nbg;
    }
    const int b = bg / p.H_kv, g = bg - b * p.H_kv;
    const long long qrs = (long long)p.H * D;      // row stride of q, o, dout, dq
    const long long krs = (long long)p.H_kv * D;   // row stride of k, v, dk, dv

    // Staging offsets: row within the tile and physical chunk of each lane.
    int qoff[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int idx = swave + NW * i;
        const int row = idx * L::ROWS_PER_LOAD + lane / L::C;
        qoff[i] = row * (int)qrs * 2 + 16 * ((lane % L::C) ^ L::dswz(row));
    }
    // Row reads (A operand of S = Q K^T and dP = dO V^T): lane (col, half)
    // reads row col (+32 for the second block), dims 16 ks + 8 half + 0..7.
    // Operand offsets. The row read of k-step ks is rbase ^ 32 ks and the
    // transposing read of block n is tbase ^ 64 n (^ T8 for its +8-row half):
    // the chunk index of a row is XOR-permuted and the row base shares no bit
    // with it. The XOR is issued at each use (lane_xor) instead of holding
    // 2 KS + 2 ND offsets in registers for the whole loop.
    const int rbase = col * L::ROWB + 16 * (half ^ L::dswz(col));
    // Transposing reads (A operand dO^T / Q^T): rows r0 and r0 + 8 of each
    // 16-row step, dims 32 n + dl .. + 3.
    int tbase;
    {
        const int r0 = 4 * half + ((lane & 15) >> 2);
        const int dl = (D >= 32 ? 16 * ((lane >> 4) & 1) : 0) + 4 * (lane & 3);
        tbase = r0 * L::ROWB + 16 * ((dl >> 3) ^ L::dswz(r0)) + 2 * (dl & 7);
    }
    // rows r0 + 8: dswz(r0 + 8) = dswz(r0) ^ (D == 16 ? 1 : 2) for every r0 < 8
    constexpr int T8 = 16 * (D == 16 ? 1 : 2) + 8 * L::ROWB;
    // (window mode keeps the plain XOR, which the compiler may hold in registers:
    // its extra per-job state leaves no registers to win)
    auto roff = [&](int ks) __attribute__((always_inline)) {
        return WINDOW ? rbase ^ (32 * ks) : lane_xor(rbase, 32 * ks);
    };
    auto toff = [&](int n, int r8) __attribute__((always_inline)) {
        const int k = 64 * n ^ (r8 ? T8 : 0);
        return WINDOW ? tbase ^ k : lane_xor(tbase, k);
    };
    const bool tzero = D < 32 && col >= D;   // D=16: rows 16..31 of dO^T / Q^T are zero
    float c;
    asm volatile("v_mov_b32 %0, %1" : "=v"(c) : "s"(p.c));

    // Window split (nslots > 0): which global key tiles this work-group
    // serves. A main work-group scans only when its own tile holds a global
    // token; a far work-group serves every eligible tile, one job each.
    int njobs = 1, elig = 0, mine = -1;
    if (WINDOW && p.nslots > 0) {
        bool scan = far;
        if (!far) {
            unsigned long long x = p.gbits[2 * tk0];
            if (2 * tk0 + 1 < p.nwords) x |= p.gbits[2 * tk0 + 1];
            scan = x != 0ull;
        }
        if (scan) {
            scan_global_tiles(p, far ? -1 : tk0, sl);
            elig = sl.nelig;
            mine = sl.mine;
        }
        if (far) {
            njobs = elig;
            if (bg == 0 && chunk == 0 && tid == 0) p.gmeta[0] = elig > 0 ? sl.end[elig - 1] : 0;
        }
    }
    const bool split_tile = !far && mine >= 0 && mine < elig;

    for (int job = 0; job < njobs; ++job) {
        if (job > 0) __syncthreads();    // every wave is done with the previous job's tiles
        const int tk = far ? sl.tile[job] : tk0;
        const int kbefore = far ? sl.before[job] : (split_tile ? sl.before[mine] : 0);
        const int k0 = tk * kBlk;
        const int wk0 = k0 + 32 * wave;
        const int key = wk0 + col;
        const bool wave_live = wk0 < T;

        // K and V rows of this lane's key as B operands: lane (col, half) holds
        // dims 16 ks + 8 half + 0..7. VL: the V rows of keys k0..k0+127 are
        // copied into v_rows instead (row r at r * ROWB, chunk c at
        // c ^ dswz(r), rows past T zero) and read with the row-read offsets;
        // KL: the K rows likewise into k_rows.
        e8_t kf[KS], vf[KS];
        {
            const long long off = ((long long)b * T + key) * krs + (long long)g * D + 8 * half;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                u32x4_t x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
                if (key < T) {
                    if (!KL) x = *(const u32x4_t *)((const unsigned short *)p.k + off + 16 * ks);
                    if (!VL) y = *(const u32x4_t *)((const unsigned short *)p.v + off + 16 * ks);
                }
                kf[ks] = __builtin_bit_cast(e8_t, x);
                vf[ks] = __builtin_bit_cast(e8_t, y);
            }
        }
        // (debug builds: the previous job's V rows read as NaN until replaced)
        lds_poison(VL && job > 0, v_rows, sizeof(v_rows), tid, kThreads);
        if (VL) {
            // two 64-row halves, each addressed from its own first row
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
                const int r0 = k0 + 64 * hb;
                if (r0 < T) {
                    const int rows = min(T - r0, 64);
                    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
                        const_cast<unsigned short *>((const unsigned short *)p.v +
                                                     ((long long)b * T + r0) * krs +
                                                     (long long)g * D),
                        (short)0, ((rows - 1) * (int)krs + D) * 2, kRsrcWord3);
                    constexpr int NL = 64 * L::ROWB / 1024;   // 1 KB loads per half
#pragma unroll
                    for (int i = 0; i < NL / 4; ++i) {
                        const int idx = wave + 4 * i;
                        const int row = idx * L::ROWS_PER_LOAD + lane / L::C;
                        const int voff = row * (int)krs * 2 + 16 * ((lane % L::C) ^ L::dswz(row));
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(
                            rv, (lds_void_t *)(v_rows + (64 * hb) * L::ROWB + idx * 1024), 16,
                            voff, 0, 0, 0);
                    }
                }
            }
        }

        if (KL) {
            // (one job: KL is not used with the window masks)
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
                const int r0 = k0 + 64 * hb;
                if (r0 < T) {
                    const int rows = min(T - r0, 64);
                    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
                        const_cast<unsigned short *>((const unsigned short *)p.k +
                                                     ((long long)b * T + r0) * krs +
                                                     (long long)g * D),
                        (short)0, ((rows - 1) * (int)krs + D) * 2, kRsrcWord3);
                    constexpr int NL = 64 * L::ROWB / 1024;   // 1 KB loads per half
#pragma unroll
                    for (int i = 0; i < NL / NW; ++i) {
                        const int idx = swave + NW * i;
                        const int row = idx * L::ROWS_PER_LOAD + lane / L::C;
                        const int koff = row * (int)krs * 2 + 16 * ((lane % L::C) ^ L::dswz(row));
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(
                            rk, (lds_void_t *)(k_rows + (64 * hb) * L::ROWB + idx * 1024), 16,
                            koff, 0, 0, 0);
                    }
                }
            }
        }

        f32x16_t dkacc[ND], dvacc[ND];
#pragma unroll
        for (int n = 0; n < ND; ++n) {
            dkacc[n] = f32x16_t{};
            dvacc[n] = f32x16_t{};
        }

        // Window mode: the global bits of this tile's 128 keys (two words) and
        // of this lane's key.
        unsigned long long gw0 = 0ull, gw1 = 0ull;
        if (WINDOW && p.gbits) {
            gw0 = p.gbits[k0 / 64];
            if (k0 / 64 + 1 < p.nwords) gw1 = p.gbits[k0 / 64 + 1];
        }
        const bool kglob = WINDOW && key < T &&
                           (((key - k0 < 64 ? gw0 : gw1) >> ((key - k0) & 63)) & 1ull);
        const bool wave_glob = WINDOW && (((wave < 2 ? gw0 : gw1) >> (32 * (wave & 1))) &
                                          0xffffffffull) != 0ull;

        // Query tiles visited, as iterations it in [itb, ite) of a list of
        // (query head, query tile) pairs: head hbase + it / nper, tile index
        // f = it % nper mapped to i_beg + f (f < nleft) or a2 + f - nleft.
        // Main work-group: the heads of its part, tiles that reach this key
        // tile (causal: rows >= k0); in window mode only those meeting the
        // band [k0 - window, k0 + 127 + window], unless the tile holds a
        // global token and is not split. Far work-group: chunk `chunk` of all
        // heads x the tiles outside the band (there only global keys are
        // visible).
        const int nqt_all = (T + BQ - 1) / BQ;
        const int i_beg = CAUSAL ? k0 / BQ : 0;
        int lo = i_beg, hi = nqt_all - 1;
        if (WINDOW && ((gw0 | gw1) == 0ull || split_tile || far)) {
            lo = (int)(max(0LL, (long long)k0 - p.window) / BQ);
            hi = (int)min((long long)nqt_all - 1, ((long long)k0 + kBlk - 1 + p.window) / BQ);
        }
        int hbase, nper, nleft = 0, a2, itb, ite;
        if (far) {
            nleft = max(0, min(lo, nqt_all) - i_beg);
            a2 = max(hi + 1, i_beg);
            nper = nleft + max(0, nqt_all - a2);
            hbase = g * p.group;
            const long long n = (long long)p.group * nper;
            itb = (int)(chunk * n / p.nchunk);
            ite = (int)((chunk + 1) * n / p.nchunk);
        } else {
            // part hs of hsplit takes a contiguous run of the key tile's (query
            // head, query tile) list; with hsplit dividing the group size the
            // runs are whole heads. A part may get no items (it then writes
            // zero sums).
            a2 = max(lo, i_beg);
            nper = hi - a2 + 1;
            hbase = g * p.group;
            const long long n = (long long)p.group * nper;
            itb = (int)(hs * n / p.hsplit);
            ite = (int)((hs + 1) * n / p.hsplit);
        }
        auto qtile0 = [&](int it, int &h) __attribute__((always_inline)) -> int {
            const int hq = it / nper;
            const int f = it - hq * nper;
            h = hbase + hq;
            return (f < nleft ? i_beg + f : a2 + (f - nleft)) * BQ;
        };

        auto stage = [&](int it, unsigned char *qd, unsigned char *od, float *sd)
            __attribute__((always_inline)) {
            int h;
            const int q0 = qtile0(it, h);
            const long long hoff = (long long)b * T * qrs + (long long)h * D;
            stage_tile<D, NW, BQ>((const unsigned short *)p.q + hoff,
                                 (const unsigned short *)p.dout + hoff, qrs, qrs, T, q0, swave, qoff,
                                 qoff, qd, od);
            if (swave < 2 && (BQ == 64 || lane < BQ)) {   // one float per lane
                const long long r = ((long long)b * p.H + h) * T + q0;
                const float *src = (swave == 0 ? p.l2 : p.delta) + r;
                const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                    const_cast<float *>(src), (short)0, min(T - q0, BQ) * 4, kRsrcWord3);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t *)(sd + BQ * swave), 4,
                                                         lane * 4, 0, 0, 0);
            }
        };

        auto compute = [&](int it, const unsigned char *qt, const unsigned char *ot,
                           const float *st) __attribute__((always_inline)) {
            int h;
            const int q0 = qtile0(it, h);
#pragma unroll
            for (int sub = 0; sub < NSUB; ++sub) {
                if (KL && sub != grp) continue;   // KL: the other group's block
                const int n0 = q0 + 32 * sub;
                if (n0 >= T || (CAUSAL && n0 + 31 < wk0)) continue;   // wave-uniform
                bool need_mask = (CAUSAL && n0 < wk0 + 31) || (wk0 + 31 >= T);
                if (WINDOW) {
                    // rows n0..n0+31 against this wave's keys wk0..wk0+31
                    const bool meets = n0 + 31 >= wk0 - p.window && n0 <= wk0 + 31 + p.window;
                    if (!meets && !wave_glob) continue;
                    const bool inside = n0 + 31 - wk0 <= p.window && wk0 + 31 - n0 <= p.window;
                    need_mask = need_mask || !inside;
                }
                // dP - Delta accumulates from C = -Delta of each row (the workspace
                // holds -Delta), so dS = P (dP - Delta) is one multiply
                f32x16_t s = f32x16_t{}, dp;
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const f32x4_t nd4 =
                        *(const lds_f32x4_t *)(st + BQ + 32 * sub + 8 * gq + 4 * half);
#pragma unroll
                    for (int e = 0; e < 4; ++e) dp[4 * gq + e] = nd4[e];
                }
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int ra = roff(ks);
                    const e8_t a = __builtin_bit_cast(
                        e8_t, *(const lds_bf16x8_t *)(qt + ra + 32 * sub * L::ROWB));
                    const e8_t a2v = __builtin_bit_cast(
                        e8_t, *(const lds_bf16x8_t *)(ot + ra + 32 * sub * L::ROWB));
                    const e8_t bv = VL ? __builtin_bit_cast(
                                             e8_t, *(const lds_bf16x8_t *)(
                                                       v_rows + 32 * wave * L::ROWB + ra))
                                       : vf[ks];
                    const e8_t bk = KL ? __builtin_bit_cast(
                                             e8_t, *(const lds_bf16x8_t *)(
                                                       k_rows + 32 * wave * L::ROWB + ra))
                                       : kf[ks];
                    s = H16::mfma(a, bk, s);
                    dp = H16::mfma(a2v, bv, dp);
                }
                // P and dS; register r is query n0 + 8(r/4) + 4half + r%4.
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const f32x4_t l4 = *(const lds_f32x4_t *)(st + 32 * sub + 8 * gq + 4 * half);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * gq + e;
                        const float pr = fast_exp2(fmaf(s[r], c, -l4[e]));
                        s[r] = pr;
                        dp[r] = pr * dp[r];
                    }
                }
                if (need_mask) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int qn = n0 + 8 * (r >> 2) + 4 * half + (r & 3);
                        bool ok = key < T && (!CAUSAL || key <= qn);
                        if (WINDOW)
                            ok = ok && ((qn - key <= p.window && key - qn <= p.window) || kglob);
                        s[r] = ok ? s[r] : 0.f;
                        dp[r] = ok ? dp[r] : 0.f;
                    }
                }
                e8_t pb[2], sb[2];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    pb[0][e] = (E)s[e];
                    pb[1][e] = (E)s[8 + e];
                    sb[0][e] = (E)dp[e];
                    sb[1][e] = (E)dp[8 + e];
                }
                int t0[ND], t1[ND];   // transposing-read offsets of this block
#pragma unroll
                for (int n = 0; n < ND; ++n) {
                    t0[n] = toff(D >= 32 ? n : 0, 0);
                    t1[n] = toff(D >= 32 ? n : 0, 1);
                }
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    const int ro = (32 * sub + 16 * s2) * L::ROWB;
#pragma unroll
                    for (int n = 0; n < ND; ++n) {
                        e8_t ao = __builtin_shufflevector(H16::read_tr(ot + t0[n] + ro),
                                                          H16::read_tr(ot + t1[n] + ro), 0,
                                                          1, 2, 3, 4, 5, 6, 7);
                        e8_t aq = __builtin_shufflevector(H16::read_tr(qt + t0[n] + ro),
                                                          H16::read_tr(qt + t1[n] + ro), 0,
                                                          1, 2, 3, 4, 5, 6, 7);
                        if (tzero) {
                            ao = e8_t{};
                            aq = e8_t{};
                        }
                        dvacc[n] = H16::mfma(ao, pb[s2], dvacc[n]);
                        dkacc[n] = H16::mfma(aq, sb[s2], dkacc[n]);
                    }
                }
            }
        };

        auto step = [&](int it, const unsigned char *qt, const unsigned char *ot, const float *st,
                        unsigned char *qn, unsigned char *on, float *sn)
            __attribute__((always_inline)) {
            __builtin_amdgcn_s_waitcnt(0);   // this lane's copies of tile `it` have landed
            __syncthreads();
            // (debug builds: the buffers about to be refilled read as NaN until then)
            lds_poison2(it + 1 < ite, qn, on, L::TILEB, tid, NT);
            lds_poison(it + 1 < ite, sn, 2 * BQ * 4, tid, NT);
            if (it + 1 < ite) stage(it + 1, qn, on, sn);
            if (wave_live) compute(it, qt, ot, st);
        };
        lds_poison2(job > 0 && itb < ite, q_lds0, o_lds0, L::TILEB, tid, NT);
        lds_poison(job > 0 && itb < ite, st_lds0, 2 * BQ * 4, tid, NT);
        if (itb < ite) stage(itb, q_lds0, o_lds0, st_lds0);
        for (int it = itb; it < ite; it += 2) {
            step(it, q_lds0, o_lds0, st_lds0, q_lds1, o_lds1, st_lds1);
            if (it + 1 < ite) step(it + 1, q_lds1, o_lds1, st_lds1, q_lds0, o_lds0, st_lds0);
        }

        if (KL) {
            // wave w + 4 (the second 32-row blocks) hands its sums to wave w (the
            // same keys) through the free tile buffers, dK then dV; every wave
            // takes every barrier (no tile copy is in flight after the last step)
            __syncthreads();
            float *mb = (float *)(wave == 0 ? q_lds0 : wave == 1 ? o_lds0
                                  : wave == 2 ? q_lds1 : o_lds1);
            static_assert(!KL || ND * 16 * 64 * 4 <= L::TILEB, "merge area");
#pragma unroll
            for (int pass = 0; pass < 2; ++pass) {
                f32x16_t *acc = pass == 0 ? dkacc : dvacc;
                if (grp == 1 && wave_live) {
#pragma unroll
                    for (int n = 0; n < ND; ++n)
#pragma unroll
                        for (int r = 0; r < 16; ++r) mb[(n * 16 + r) * 64 + lane] = acc[n][r];
                }
                __syncthreads();
                if (grp == 0 && wave_live) {
#pragma unroll
                    for (int n = 0; n < ND; ++n)
#pragma unroll
                        for (int r = 0; r < 16; ++r) acc[n][r] += mb[(n * 16 + r) * 64 + lane];
                }
                __syncthreads();
            }
        }
        if (wave_live && key < T && grp == 0) {
            // dK^T / dV^T register r of block n is dim 32n + 8(r/4) + 4half + r%4.
            const long long off = ((long long)b * T + key) * krs + (long long)g * D;
            if (far) {
                // nothing for the tile's other keys: they see no far query
            } else if (p.hsplit > 1) {
                // this part's fp32 sums; the reduce kernel adds the parts and scales dK
                const long long poff = (long long)hs * p.B * T * krs + off;
#pragma unroll
                for (int n = 0; n < ND; ++n)
#pragma unroll
                    for (int rg = 0; rg < 4; ++rg) {
                        const int d = 32 * n + 8 * rg + 4 * half;
                        if (D >= 32 || d < D) {
                            f32x4_t k4, v4;
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                k4[e] = dkacc[n][4 * rg + e];
                                v4[e] = dvacc[n][4 * rg + e];
                            }
                            *(f32x4_t *)(p.dkpart + poff + d) = k4;
                            *(f32x4_t *)(p.dvpart + poff + d) = v4;
                        }
                    }
            } else {
                unsigned short *dkrow = (unsigned short *)p.dk + off;
                unsigned short *dvrow = (unsigned short *)p.dv + off;
                const float sc = p.scale;
#pragma unroll
                for (int n = 0; n < ND; ++n)
#pragma unroll
                    for (int rg = 0; rg < 4; ++rg) {
                        const int d = 32 * n + 8 * rg + 4 * half;
                        if (D >= 32 || d < D) {
                            e4_t k4, v4;
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                k4[e] = (E)(dkacc[n][4 * rg + e] * sc);
                                v4[e] = (E)dvacc[n][4 * rg + e];
                            }
                            *(u32x2_t *)(dkrow + d) = __builtin_bit_cast(u32x2_t, k4);
                            *(u32x2_t *)(dvrow + d) = __builtin_bit_cast(u32x2_t, v4);
                        }
                    }
            }
            if (WINDOW && kglob && (far || split_tile)) {
                // A global key of a split tile: this part's fp32 sums (dK
                // unscaled) go to its slot, rank = global keys before it.
                const int kk = key - k0;
                const int rank = kbefore + (kk < 64 ? __popcll(gw0 & ((1ull << kk) - 1ull))
                                                    : __popcll(gw0) +
                                                          __popcll(gw1 & ((1ull << (kk - 64)) - 1ull)));
                const int part = far ? p.hsplit + chunk : hs;
                const long long goff = (((long long)rank * p.nparts + part) * nbg + bg) * D;
#pragma unroll
                for (int n = 0; n < ND; ++n)
#pragma unroll
                    for (int rg = 0; rg < 4; ++rg) {
                        const int d = 32 * n + 8 * rg + 4 * half;
                        if (D >= 32 || d < D) {
                            f32x4_t k4, v4;
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                k4[e] = dkacc[n][4 * rg + e];
                                v4[e] = dvacc[n][4 * rg + e];
                            }
                            *(f32x4_t *)(p.gpk + goff + d) = k4;
                            *(f32x4_t *)(p.gpv + goff + d) = v4;
                        }
                    }
                if (far && bg == 0 && chunk == 0 && half == 0) p.gmeta[4 + rank] = key;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// dQ. Work-group: query rows [q0, q0 + 128) of head h of batch b, heaviest
// causal tiles first; wave w owns rows wq0 = q0 + 32w .. + 31 (lane col = row
// wq0 + col). Key tiles of 64: K (dual swizzle: read as rows for S^T and
// transposed for dQ^T) and V (row reads only) in LDS, two buffers.
// S^T = K Q^T and dP^T = V dO^T put one query per lane column, so the row's
// L2 and Delta are per-lane scalars; register r of block kb is key
// key0 + 32 kb + 8(r/4) + 4half + r%4.
// ---------------------------------------------------------------------------
template <typename E, int D, bool CAUSAL, bool WINDOW, bool G2 = false>
__global__ __launch_bounds__(G2 ? 2 * kThreads : kThreads) void fa_bwd_dq_kernel(BwdParams p) {
    using L = Bf16Layout<D>;
    using H16 = Half16<E>;
    typedef typename H16::v8 e8_t;
    typedef typename H16::v4 e4_t;
    constexpr int BK = L::BK;
    constexpr int KS = D / 16;
    constexpr int ND = (D + 31) / 32;
    constexpr int NV = D >= 32 ? D / 32 : 1;
    constexpr int NI = (L::NLOAD + 3) / 4;
    static_assert(!G2 || (!WINDOW && D >= 32), "G2: plain masks, D >= 32");

    // With G2 (8 waves, two key-range groups of 4) each variable holds both
    // groups' buffers, group g at offset g * TILEB.
    constexpr int NG = G2 ? 2 : 1;
    __shared__ __attribute__((aligned(1024))) unsigned char k_lds0_[NG * L::TILEB];
    __shared__ __attribute__((aligned(1024))) unsigned char v_lds0_[NG * L::TILEB];
    __shared__ __attribute__((aligned(1024))) unsigned char k_lds1_[NG * L::TILEB];
    __shared__ __attribute__((aligned(1024))) unsigned char v_lds1_[NG * L::TILEB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave8 = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = G2 ? (wave8 >> 2) : 0;
    const int wave = G2 ? (wave8 & 3) : wave8;
    unsigned char *const k_lds0 = k_lds0_ + grp * L::TILEB;
    unsigned char *const v_lds0 = v_lds0_ + grp * L::TILEB;
    unsigned char *const k_lds1 = k_lds1_ + grp * L::TILEB;
    unsigned char *const v_lds1 = v_lds1_ + grp * L::TILEB;
    const int col = lane & 31, half = lane >> 5;
    const int T = p.T;
    const int nbh = p.B * p.H;
    const int npart = G2 ? p.dq_parts : 1;
    const int kpart = G2 ? (int)(blockIdx.x % npart) : 0;   // this work-group's key part
    const int id = G2 ? (int)(blockIdx.x / npart) : (int)blockIdx.x;
    const int tq = id / nbh;
    const int bh = id - tq * nbh;
    const int b = bh / p.H, h = bh - b * p.H;
    const int g = h / p.group;
    const int q0 = (p.nblk - 1 - tq) * kBlk;
    const int wq0 = q0 + 32 * wave;
    const int qrow = wq0 + col;
    const bool wave_live = wq0 < T;
    const long long qrs = (long long)p.H * D;
    const long long krs = (long long)p.H_kv * D;
    const unsigned short *kbase = (const unsigned short *)p.k + (long long)b * T * krs + g * D;
    const unsigned short *vbase = (const unsigned short *)p.v + (long long)b * T * krs + g * D;

    // Q and dO rows of this lane's query as B operands.
    e8_t qf[KS], df[KS];
    {
        const long long off = ((long long)b * T + qrow) * qrs + (long long)h * D + 8 * half;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4_t x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
            if (qrow < T) {
                x = *(const u32x4_t *)((const unsigned short *)p.q + off + 16 * ks);
                y = *(const u32x4_t *)((const unsigned short *)p.dout + off + 16 * ks);
            }
            qf[ks] = __builtin_bit_cast(e8_t, x);
            df[ks] = __builtin_bit_cast(e8_t, y);
        }
    }
    // Delta = dO . O of this lane's row (the two halves of the row live in
    // lanes col and col + 32) and L2 = L log2(e): used here and stored in the
    // workspace for the dK/dV kernel, which runs after this one.
    float l2 = 0.f, dl = 0.f;
    {
        const long long off = ((long long)b * T + qrow) * qrs + (long long)h * D + 8 * half;
        float part = 0.f;
        if (qrow < T) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const e8_t ov = __builtin_bit_cast(
                    e8_t, *(const u32x4_t *)((const unsigned short *)p.o + off + 16 * ks));
#pragma unroll
                for (int e = 0; e < 8; ++e) part = fmaf((float)ov[e], (float)df[ks][e], part);
            }
        }
        dl = half_swap_sum(part);
        if (qrow < T) {
            const long long r = ((long long)b * p.H + h) * T + qrow;
            l2 = p.lse[r] * kLog2e;
            if (half == 0 && grp == 0 && kpart == 0) {
                p.delta[r] = -dl;   // the dK/dV kernel starts its dP sums from it
                p.l2[r] = l2;
            }
        }
    }

    const int kend = CAUSAL ? min(T, q0 + kBlk) : T;
    const int nkt = (kend + BK - 1) / BK;
    // G2: this part's key tiles [pbeg, pend); group 0 takes the first ghalf
    // of them, group 1 the rest.
    const int pbeg = (int)((long long)kpart * nkt / npart);
    const int pend = (int)((long long)(kpart + 1) * nkt / npart);
    const int ghalf = (pend - pbeg + 1) / 2;
    const int jbeg = G2 ? (grp ? pbeg + ghalf : pbeg) : 0;
    const int jend = G2 ? (grp ? pend : pbeg + ghalf) : nkt;
    // Window mode: key tiles meeting the band of this query tile (blo..bhi)
    // or holding a global token; the others are never loaded.
    int blo = 0, bhi = nkt - 1;
    if (WINDOW) {
        const long long q1 = min(q0 + kBlk, T) - 1;
        blo = (int)(max(0LL, (long long)q0 - p.window) / BK);
        bhi = (int)(min((long long)kend - 1, q1 + p.window) / BK);
    }
    auto next_tile = [&](int j) __attribute__((always_inline)) -> int {
        int t = j + 1;
        if (!WINDOW) return t;
        const unsigned long long *gbits = p.gbits;
        if (t < blo) return gbits ? first_nonzero_word(gbits, t, blo) : blo;
        if (t <= bhi) return t;
        return gbits ? first_nonzero_word(gbits, t, nkt) : max(t, nkt);
    };
    // read between steps, never after a step's prefetch is issued
    auto tile_bits = [&](int t) __attribute__((always_inline)) -> unsigned long long {
        return (WINDOW && p.gbits && t < nkt) ? p.gbits[t] : 0ull;
    };

    int koff[NI], voff[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int idx = wave + 4 * i;
        const int row = idx * L::ROWS_PER_LOAD + lane / L::C;
        const int pc = lane % L::C;
        koff[i] = row * (int)krs * 2 + 16 * (pc ^ L::dswz(row));
        voff[i] = row * (int)krs * 2 + 16 * (pc ^ L::kswz(row));
    }
    int kaddr[KS], vaddr[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        kaddr[ks] = col * L::ROWB + 16 * ((2 * ks + half) ^ L::dswz(col));
        vaddr[ks] = col * L::ROWB + 16 * ((2 * ks + half) ^ L::kswz(col));
    }
    int taddr[NV], taddr8[NV];
    {
        const int r0 = 4 * half + ((lane & 15) >> 2);
        const int dl4 = (D >= 32 ? 16 * ((lane >> 4) & 1) : 0) + 4 * (lane & 3);
#pragma unroll
        for (int n = 0; n < NV; ++n) {
            const int d = 32 * n + dl4;
            taddr[n] = r0 * L::ROWB + 16 * ((d >> 3) ^ L::dswz(r0)) + 2 * (d & 7);
            taddr8[n] = (r0 + 8) * L::ROWB + 16 * ((d >> 3) ^ L::dswz(r0 + 8)) + 2 * (d & 7);
        }
    }
    const bool tzero = D < 32 && col >= D;

    f32x16_t dqacc[ND];
#pragma unroll
    for (int n = 0; n < ND; ++n) dqacc[n] = f32x16_t{};
    float c;
    asm volatile("v_mov_b32 %0, %1" : "=v"(c) : "s"(p.c));

    auto tile = [&](bool need_mask, int j, const unsigned char *kt, const unsigned char *vt,
                    unsigned long long gb) __attribute__((always_inline)) {
        const int key0 = j * BK;
        f32x16_t s0 = f32x16_t{}, s1 = f32x16_t{}, d0 = f32x16_t{}, d1 = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const e8_t a0 = __builtin_bit_cast(e8_t, *(const lds_bf16x8_t *)(kt + kaddr[ks]));
            const e8_t a1 =
                __builtin_bit_cast(e8_t, *(const lds_bf16x8_t *)(kt + kaddr[ks] + 32 * L::ROWB));
            const e8_t b0 = __builtin_bit_cast(e8_t, *(const lds_bf16x8_t *)(vt + vaddr[ks]));
            const e8_t b1 =
                __builtin_bit_cast(e8_t, *(const lds_bf16x8_t *)(vt + vaddr[ks] + 32 * L::ROWB));
            s0 = H16::mfma(a0, qf[ks], s0);
            s1 = H16::mfma(a1, qf[ks], s1);
            d0 = H16::mfma(b0, df[ks], d0);
            d1 = H16::mfma(b1, df[ks], d1);
        }
        // P^T and dS^T in place of S^T (s0, s1).
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float p0 = fast_exp2(fmaf(s0[r], c, -l2));
            const float p1 = fast_exp2(fmaf(s1[r], c, -l2));
            s0[r] = p0 * (d0[r] - dl);
            s1[r] = p1 * (d1[r] - dl);
        }
        if (need_mask) {
            const int lim = (CAUSAL ? min(qrow, T - 1) : T - 1) - key0 - 4 * half;
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
                    s0[r] = v0 ? s0[r] : 0.f;
                    s1[r] = v1 ? s1[r] : 0.f;
                }
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int off = 8 * (r >> 2) + (r & 3);
                    s0[r] = off <= lim ? s0[r] : 0.f;
                    s1[r] = off + 32 <= lim ? s1[r] : 0.f;
                }
            }
        }
        // dS^T as the B operand: k-step s4 covers keys 16 s4 + 8(e/4) + 4half + e%4.
        e8_t sb[4];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            sb[0][e] = (E)s0[e];
            sb[1][e] = (E)s0[8 + e];
            sb[2][e] = (E)s1[e];
            sb[3][e] = (E)s1[8 + e];
        }
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
#pragma unroll
            for (int n = 0; n < ND; ++n) {
                const int tn = D >= 32 ? n : 0;
                const int ro = 16 * s4 * L::ROWB;
                e8_t a = __builtin_shufflevector(H16::read_tr(kt + taddr[tn] + ro),
                                                 H16::read_tr(kt + taddr8[tn] + ro), 0, 1, 2, 3,
                                                 4, 5, 6, 7);
                if (tzero) a = e8_t{};
                dqacc[n] = H16::mfma(a, sb[s4], dqacc[n]);
            }
        }
    };

    auto step = [&](int j, unsigned long long gb, int jn, const unsigned char *kt,
                    const unsigned char *vt, unsigned char *kn, unsigned char *vn)
        __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        // (debug builds: the buffers about to be refilled read as NaN until then;
        // with G2 each group fills its own)
        lds_poison2(jn < jend, kn, vn, L::TILEB, G2 ? (tid & (kThreads - 1)) : tid, kThreads);
        if (jn < jend)
            stage_tile<D>(kbase, vbase, krs, krs, T, jn * BK, wave, koff, voff, kn, vn);
        const int key0 = j * BK;
        bool active = wave_live && (!CAUSAL || key0 <= wq0 + 31) && (!G2 || j < jend);
        bool need_mask = (key0 + BK > T) || (CAUSAL && key0 + BK - 1 > wq0);
        if (WINDOW) {
            const long long wlo = (long long)wq0 - p.window, whi = (long long)wq0 + 31 + p.window;
            const bool meets = key0 + BK - 1 >= wlo && key0 <= whi;
            const bool inside = key0 >= (long long)wq0 + 31 - p.window &&
                                key0 + BK - 1 <= (long long)wq0 + p.window;
            active = active && (meets || gb != 0ull);
            need_mask = need_mask || !inside;
        }
        if (active) tile(need_mask, j, kt, vt, gb);
    };
    if (G2) {
        // both groups take ghalf steps, one barrier each; group 1's last step is
        // idle when nkt is odd
        if (jbeg < jend)
            stage_tile<D>(kbase, vbase, krs, krs, T, jbeg * BK, wave, koff, voff, k_lds0, v_lds0);
        for (int i = 0; i < ghalf; i += 2) {
            step(jbeg + i, 0ull, jbeg + i + 1, k_lds0, v_lds0, k_lds1, v_lds1);
            if (i + 1 < ghalf)
                step(jbeg + i + 1, 0ull, jbeg + i + 2, k_lds1, v_lds1, k_lds0, v_lds0);
        }
        // wave w + 4 leaves its dQ^T accumulators in LDS, lane-major; wave w
        // (the same 32 rows) adds them after its own. Every wave takes both
        // barriers; after the first, all K/V reads are done.
        static_assert(!G2 || ND * 16 * 64 * 4 <= NG * L::TILEB, "merge area");
        __syncthreads();
        float *mb = (float *)(wave == 0 ? k_lds0_ : wave == 1 ? v_lds0_
                              : wave == 2 ? k_lds1_ : v_lds1_);
        if (grp == 1 && wave_live) {
#pragma unroll
            for (int n = 0; n < ND; ++n)
#pragma unroll
                for (int r = 0; r < 16; ++r) mb[(n * 16 + r) * 64 + lane] = dqacc[n][r];
        }
        __syncthreads();
        if (grp == 1) return;
        if (wave_live) {
#pragma unroll
            for (int n = 0; n < ND; ++n)
#pragma unroll
                for (int r = 0; r < 16; ++r) dqacc[n][r] += mb[(n * 16 + r) * 64 + lane];
        }
    } else {
        int j = next_tile(-1);
        unsigned long long gj = tile_bits(j);
        if (j < nkt)
            stage_tile<D>(kbase, vbase, krs, krs, T, j * BK, wave, koff, voff, k_lds0, v_lds0);
        while (j < nkt) {
            const int jn = next_tile(j);
            const unsigned long long gn = tile_bits(jn);
            step(j, gj, jn, k_lds0, v_lds0, k_lds1, v_lds1);
            if (jn >= nkt) break;
            const int jnn = next_tile(jn);
            const unsigned long long gnn = tile_bits(jnn);
            step(jn, gn, jnn, k_lds1, v_lds1, k_lds0, v_lds0);
            j = jnn;
            gj = gnn;
        }
    }

    if (!wave_live || qrow >= T) return;
    if (G2 && npart > 1) {
        // this part's fp32 sums; fa_bwd_dq_reduce_kernel adds the parts and scales
        float *prow = p.dqpart + ((long long)kpart * p.B * T + (long long)b * T + qrow) * qrs +
                      (long long)h * D;
#pragma unroll
        for (int n = 0; n < ND; ++n)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int d = 32 * n + 8 * rg + 4 * half;
                f32x4_t q4;
#pragma unroll
                for (int e = 0; e < 4; ++e) q4[e] = dqacc[n][4 * rg + e];
                *(f32x4_t *)(prow + d) = q4;
            }
        return;
    }
    unsigned short *dqrow = (unsigned short *)p.dq + ((long long)b * T + qrow) * qrs + h * D;
    const float sc = p.scale;
#pragma unroll
    for (int n = 0; n < ND; ++n)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            const int d = 32 * n + 8 * rg + 4 * half;
            if (D >= 32 || d < D) {
                e4_t q4;
#pragma unroll
                for (int e = 0; e < 4; ++e) q4[e] = (E)(dqacc[n][4 * rg + e] * sc);
                *(u32x2_t *)(dqrow + d) = __builtin_bit_cast(u32x2_t, q4);
            }
        }
}

// ---------------------------------------------------------------------------
// dK, dV from the head-split parts: dK = scale * sum_s dkpart[s], dV =
// sum_s dvpart[s], parts added in order s = 0, 1, ... (deterministic). Each
// thread handles four consecutive elements of the [B][T][H_kv][D] arrays.
// ---------------------------------------------------------------------------
template <typename E>
__global__ __launch_bounds__(256) void fa_bwd_reduce_kernel(BwdParams p, long long n) {
    typedef E e4v __attribute__((ext_vector_type(4)));
    // n = B * T * H_kv * D elements per part, a multiple of 4
    const long long i = ((long long)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= n) return;
    f32x4_t k = {0.f, 0.f, 0.f, 0.f}, v = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < p.hsplit; ++s) {
        k += *(const f32x4_t *)(p.dkpart + s * n + i);
        v += *(const f32x4_t *)(p.dvpart + s * n + i);
    }
    e4v k4, v4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        k4[e] = (E)(k[e] * p.scale);
        v4[e] = (E)v[e];
    }
    *(e4v *)((E *)p.dk + i) = k4;
    *(e4v *)((E *)p.dv + i) = v4;
}

// ---------------------------------------------------------------------------
// Global keys of split tiles: dK = scale * sum_part gpk[slot][part], dV =
// sum_part gpv[slot][part], parts in order (deterministic), over the rows the
// other kernels wrote for those keys. Thread: (slot, b, g, 4 dims).
// ---------------------------------------------------------------------------
// dQ = scale * sum_s dqpart[s], parts added in order s = 0, 1, ... Each thread
// handles four consecutive elements of the [B][T][H][D] array.
template <typename E>
__global__ __launch_bounds__(256) void fa_bwd_dq_reduce_kernel(BwdParams p, long long n) {
    typedef E e4v __attribute__((ext_vector_type(4)));
    const long long i = ((long long)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= n) return;
    f32x4_t q = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < p.dq_parts; ++s) q += *(const f32x4_t *)(p.dqpart + s * n + i);
    e4v q4;
#pragma unroll
    for (int e = 0; e < 4; ++e) q4[e] = (E)(q[e] * p.scale);
    *(e4v *)((E *)p.dq + i) = q4;
}

template <typename E>
__global__ __launch_bounds__(256) void fa_bwd_gsum_kernel(BwdParams p, int D) {
    typedef E e4v __attribute__((ext_vector_type(4)));
    const int nbg = p.B * p.H_kv;
    const long long per = (long long)nbg * (D / 4);
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long r = i / per;
    if (r >= p.gmeta[0] || r >= p.nslots) return;
    const int key = p.gmeta[4 + r];
    if (key < 0 || key >= p.T) return;
    const int rest = (int)(i - r * per);
    const int bg = rest / (D / 4);
    const int d = 4 * (rest - bg * (D / 4));
    const int b = bg / p.H_kv, g = bg - b * p.H_kv;
    f32x4_t k = {0.f, 0.f, 0.f, 0.f}, v = {0.f, 0.f, 0.f, 0.f};
    for (int part = 0; part < p.nparts; ++part) {
        const long long off = ((r * p.nparts + part) * nbg + bg) * D + d;
        k += *(const f32x4_t *)(p.gpk + off);
        v += *(const f32x4_t *)(p.gpv + off);
    }
    e4v k4, v4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        k4[e] = (E)(k[e] * p.scale);
        v4[e] = (E)v[e];
    }
    const long long o = (((long long)b * p.T + key) * p.H_kv + g) * D + d;
    *(e4v *)((E *)p.dk + o) = k4;
    *(e4v *)((E *)p.dv + o) = v4;
}

// ---------------------------------------------------------------------------
// Host side: validation (no HIP calls), launch.
// ---------------------------------------------------------------------------
constexpr long long kMaxElems = 1LL << 62;
constexpr long long kMaxGridB = (1LL << 24) - 1;

bool aligned16(const void *ptr) { return ((uintptr_t)ptr % 16) == 0; }

constexpr long long kTargetWG = 1024;   // dK/dV work-groups aimed for (4 per CU)
constexpr long long kNumCUB = 256;      // MI355X compute units
constexpr long long kMaxQueryParts = 8; // query-tile runs per key tile (library choice)

// Parts of the dK/dV kernel: the requested count (capped at the group size)
// or, for 0, enough parts to bring the launch to kTargetWG work-groups --
// runs of query heads, or, with one query head per kv head, key tiles for at
// most half the CUs and T >= 4096, runs of each key tile's query tiles (not
// for the window masks, whose key tiles see only their band's query tiles);
// at D = 128 no more than keep the launch within two work-groups per CU.
// The D = 128 dK/dV variant with V rows in LDS and 32-row query tiles (two
// work-groups per CU) for plain masks, except for long rows with two or more
// work-groups of whole key tiles per CU already, where 64-row tiles' lower
// per-step cost wins (measured on MI355X, bf16 causal: B=64 T=1024 88 vs 95
// us, B=16 H_kv=4 T=2048 975 vs 1099 us, B=1 T=8192 116 vs 118 us; but
// B=8 T=8192 522 vs 505 us).
bool dkdv_vlds(int B, int H_kv, int T, int D, bool window) {
    if (D != 128 || window) return false;
    const long long units = mul_sat(mul_sat(B, H_kv), ((long long)T + kBlk - 1) / kBlk);
    return !(T >= 4096 && units >= 2 * kNumCUB);
}

// The D = 128 dK/dV variant with K rows in LDS and 8-wave work-groups (one per
// CU, two waves per SIMD, 64-row query tiles) for plain masks when the launch
// has at most two work-groups per CU (measured on MI355X, bf16 causal backward,
// against the choice above: B=8 T=8192 498 -> 458 us, B=4 T=8192 465 -> 372,
// B=16 T=2048 129 -> 107, B=1 T=8192 120 -> 116, B=64 T=1024 91 -> 90; with
// 1024 work-groups it lost: B=2 T=8192 in 8 query-tile runs 197 -> 212, B=16
// H=16 H_kv=4 T=2048 1004 -> 1026).
bool dkdv_klds(long long workgroups, int D, bool window) {
    return D == 128 && !window && workgroups <= 2 * kNumCUB;
}

int head_parts(int B, int H, int H_kv, int T, int D, int requested, bool window) {
    const int group = H / H_kv;
    if (requested > 0) return requested < group ? requested : group;
    const long long nwg = mul_sat(mul_sat(B, H_kv), ((long long)T + kBlk - 1) / kBlk);
    if (nwg <= 0) return 1;
    const long long want = nwg >= kTargetWG ? 1 : (kTargetWG + nwg - 1) / nwg;
    // one query head per kv head, key tiles for at most half the CUs and long
    // rows: split each key tile's query tiles instead (at most kMaxQueryParts
    // runs; shorter rows or more key tiles lose more to the parts' fp32
    // traffic than they gain)
    // D = 128, plain masks: no more parts than keep the launch within two
    // work-groups per CU, where the 8-wave dK/dV kernel runs (dkdv_klds; measured
    // on MI355X, bf16 causal backward: B=2 T=8192 in 4 query-tile runs instead
    // of 8 195 -> 178 us, B=4 H=16 H_kv=1 T=4096 with 4 head parts instead of 8
    // 938 -> 916 us)
    long long cap = want;
    if (D == 128 && !window && nwg <= 2 * kNumCUB) {
        const long long fit = (2 * kNumCUB) / nwg;
        cap = fit < want ? fit : want;
    }
    if (!window && group == 1 && nwg <= kNumCUB / 2 && T >= 4096)
        return (int)(cap < kMaxQueryParts ? cap : kMaxQueryParts);
    return (int)(cap < group ? cap : group);
}

// Workspace: -Delta and L2 (B*H*T floats each, padded to 16 bytes), then, with
// hs > 1 head parts, the fp32 dK and dV parts (hs * B*T*H_kv*D floats each).
// Sets *stat_bytes to the size of the first region; -1 on overflow.
long long bwd_ws_bytes(int B, int H, int H_kv, int T, int D, int hs, int dqp,
                       long long *stat_bytes, long long *dq_offset) {
    long long rows, part, total, dqb;
    if (__builtin_mul_overflow((long long)B * H, (long long)T, &rows) || rows > (1LL << 58))
        return -1;
    const long long stat = (rows * 8 + 15) / 16 * 16;
    if (stat_bytes) *stat_bytes = stat;
    total = stat;
    if (hs > 1) {
        if (__builtin_mul_overflow((long long)B * T, (long long)H_kv * D, &part) ||
            __builtin_mul_overflow(part, (long long)hs * 8, &part) ||
            __builtin_add_overflow(total, part, &total))
            return -1;
    }
    if (dq_offset) *dq_offset = total;
    if (dqp > 1) {
        if (__builtin_mul_overflow(rows, (long long)D, &dqb) ||
            __builtin_mul_overflow(dqb, (long long)dqp * 4, &dqb) ||
            __builtin_add_overflow(total, dqb, &total))
            return -1;
    }
    return total;
}

// Two key-range groups in the dQ kernel on small grids, plain masks only. At
// D = 128 the forward's rule: at most a quarter of the 512 resident 4-wave
// work-groups (256 CUs x 2 by registers), or rows of >= 2048 keys with all of
// them resident. At D = 64 (768 resident: 3 per CU by registers) at most a
// quarter, or half with rows of >= 2048 keys (with all resident it was 5 %
// slower).
int dq_groups_for(int B, int H, int T, int D, bool window) {
    const long long units = mul_sat(mul_sat(B, H), ((long long)T + kBlk - 1) / kBlk);
    if (window || D < 64) return 1;
    if (D == 64) return units <= 768 / 4 || (T >= 2048 && units <= 768 / 2) ? 2 : 1;
    return units <= 512 / 4 || (T >= 2048 && units <= 512) ? 2 : 1;
}

// Key parts of the two-group dQ kernel: with rows of >= 4096 keys and query
// tiles for at most half the CUs (one 8-wave work-group per CU), enough parts
// to give each CU one work-group (at most 8).
int dq_parts_for(int B, int H, int T, int D, bool window) {
    if (dq_groups_for(B, H, T, D, window) != 2 || T < 4096) return 1;
    const long long units = mul_sat(mul_sat(B, H), ((long long)T + kBlk - 1) / kBlk);
    if (units <= 0 || units > kNumCUB / 2) return 1;
    const long long n = kNumCUB / units;
    return (int)(n < 8 ? n : 8);
}

// Far parts per split global tile: runs of about the main work-group's
// iteration count (its heads x the band's query tiles) over all heads x all
// query tiles.
int far_chunks(int T, int window, int group, int hs) {
    const long long nqt = ((long long)T + 63) / 64;
    const long long nband = ((long long)kBlk + 2LL * window) / 64 + 2;
    const long long nh = (group + hs - 1) / hs;
    long long run = nh * nband;
    if (run < 4) run = 4;
    long long n = ((long long)group * nqt + run - 1) / run;
    if (n < 1) n = 1;
    return (int)(n < 256 ? n : 256);
}

// Bytes of the window split region for `slots` global-key slots: a 16-byte
// header, the slot -> key map (padded to 16 bytes), then gpk and gpv.
long long split_bytes(long long slots, int nparts, int B, int H_kv, int D) {
    if (slots <= 0) return 0;
    long long per, map = (slots * 4 + 15) / 16 * 16, total;
    if (__builtin_mul_overflow((long long)nparts * B, (long long)H_kv * D * 8, &per) ||
        __builtin_mul_overflow(per, slots, &total) || __builtin_add_overflow(total, 16 + map, &total))
        return -1;
    return total;
}

// dQ first: it also writes -Delta and L2, which the dK/dV kernel reads. The
// global-key sums go last, over the rows the dK/dV (or reduce) kernel wrote.
template <typename E, int D, bool CAUSAL, bool WINDOW>
hipError_t launch_bwd(const BwdParams &p, hipStream_t s) {
    constexpr bool CAN_G2 = D >= 64 && !WINDOW;
    hipError_t e;
    if (CAN_G2 && p.dq_groups == 2)
        e = launch_kernel((fa_bwd_dq_kernel<E, D, CAUSAL, WINDOW, CAN_G2>),
                          dim3((unsigned)((long long)p.B * p.H * p.nblk * p.dq_parts)),
                          dim3(2 * kThreads), s, p);
    else
        e = launch_kernel((fa_bwd_dq_kernel<E, D, CAUSAL, WINDOW>),
                          dim3((unsigned)((long long)p.B * p.H * p.nblk)), dim3(kThreads), s, p);
    if (e != hipSuccess) return e;
    constexpr bool CAN_VL = D == 128 && !WINDOW;
    const dim3 grid((unsigned)((long long)p.B * p.H_kv * p.nblk * p.hsplit + p.nfar));
    if (CAN_VL && p.klds)
        e = launch_kernel((fa_bwd_dkdv_kernel<E, D, CAUSAL, WINDOW, false, CAN_VL>), grid,
                          dim3(2 * kThreads), s, p);
    else if (CAN_VL && p.vlds)
        e = launch_kernel((fa_bwd_dkdv_kernel<E, D, CAUSAL, WINDOW, CAN_VL>), grid, dim3(kThreads),
                          s, p);
    else
        e = launch_kernel((fa_bwd_dkdv_kernel<E, D, CAUSAL, WINDOW>), grid, dim3(kThreads), s, p);
    if (e != hipSuccess) return e;
    if (p.hsplit > 1) {
        const long long n = (long long)p.B * p.T * p.H_kv * D;
        e = launch_kernel((fa_bwd_reduce_kernel<E>), dim3((unsigned)((n / 4 + 255) / 256)),
                          dim3(256), s, p, n);
        if (e != hipSuccess) return e;
    }
    if (p.dq_parts > 1) {
        const long long n = (long long)p.B * p.T * p.H * D;
        e = launch_kernel((fa_bwd_dq_reduce_kernel<E>), dim3((unsigned)((n / 4 + 255) / 256)),
                          dim3(256), s, p, n);
        if (e != hipSuccess) return e;
    }
    if (WINDOW && p.nslots > 0) {
        const long long n = (long long)p.nslots * p.B * p.H_kv * (D / 4);
        e = launch_kernel((fa_bwd_gsum_kernel<E>), dim3((unsigned)((n + 255) / 256)), dim3(256),
                          s, p, D);
    }
    return e;
}

template <typename E, bool CAUSAL, bool WINDOW>
hipError_t launch_bwd_d(const BwdParams &p, int D, hipStream_t s) {
    switch (D) {
        case 16: return launch_bwd<E, 16, CAUSAL, WINDOW>(p, s);
        case 32: return launch_bwd<E, 32, CAUSAL, WINDOW>(p, s);
        case 64: return launch_bwd<E, 64, CAUSAL, WINDOW>(p, s);
        default: return launch_bwd<E, 128, CAUSAL, WINDOW>(p, s);
    }
}

template <typename E, bool WINDOW>
hipError_t launch_bwd_c(const BwdParams &p, int D, int causal, hipStream_t s) {
    return causal ? launch_bwd_d<E, true, WINDOW>(p, D, s) : launch_bwd_d<E, false, WINDOW>(p, D, s);
}

}  // namespace

extern "C" long long fa_bwd_workspace_bytes(int B, int H, int H_kv, int T, int D,
                                            int head_split) {
    if (B < 0 || H < 1 || H_kv < 1 || T < 0 || H % H_kv != 0 || head_split < 0 ||
        (D != 16 && D != 32 && D != 64 && D != 128))
        return -1;
    return bwd_ws_bytes(B, H, H_kv, T, D, head_parts(B, H, H_kv, T, D, head_split, false),
                        dq_parts_for(B, H, T, D, false), nullptr, nullptr);
}

extern "C" long long fa_bwd_window_workspace_bytes(int B, int H, int H_kv, int T, int D,
                                                   int window, int n_global, int head_split) {
    const long long base = fa_bwd_workspace_bytes(B, H, H_kv, T, D, head_split);
    if (base < 0 || window < 0 || n_global < 0) return -1;
    if (n_global == 0 || T == 0 || B == 0) return base;
    const int hs = head_parts(B, H, H_kv, T, D, head_split, true);
    const int w = window < T ? window : T;
    const long long slots = n_global < T ? n_global : T;
    const long long extra =
        split_bytes(slots, hs + far_chunks(T, w, H / H_kv, hs), B, H_kv, D);
    long long total;
    if (extra < 0 || __builtin_add_overflow(base, extra, &total)) return -1;
    return total;
}

namespace {

// Validation and launch shared by fa_bwd (window < 0) and fa_bwd_window.
int bwd_impl(const void *q, const void *k, const void *v, const void *o, const float *lse,
             const void *dout, void *dq, void *dk, void *dv, int B, int H, int H_kv, int T,
             int D, int causal, float scale, int dtype, int window, const void *global_bits,
             int head_split, void *workspace, long long workspace_bytes, void *stream) {
    if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16)
        return FA_ERR_DTYPE;
    if (dtype == FA_DTYPE_F32) return FA_ERR_DTYPE;   // 16-bit MFMA kernels only
    if (B < 0 || T < 0 || H < 1 || H_kv < 1 || head_split < 0) return FA_ERR_BAD_SHAPE;
    if (H % H_kv != 0) return FA_ERR_HEADS;
    if (D != 16 && D != 32 && D != 64 && D != 128) return FA_ERR_HEAD_DIM;
    if (!isfinite(scale) || !isfinite(scale * kLog2e)) return FA_ERR_SCALE;
    if (B == 0 || T == 0) return FA_OK;
    if (T > (1 << 30)) return FA_ERR_OVERFLOW;   // 32-bit row arithmetic in the kernels
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !workspace)
        return FA_ERR_NULL_PTR;
    const void *ptrs[] = {q, k, v, o, dout, dq, dk, dv, workspace};
    for (const void *ptr : ptrs)
        if (!aligned16(ptr)) return FA_ERR_ALIGN;
    if (((uintptr_t)lse % 4) != 0 || ((uintptr_t)global_bits % 8) != 0) return FA_ERR_ALIGN;
    const int hs = head_parts(B, H, H_kv, T, D, head_split, window >= 0);
    // The workspace starts with fa_bwd's layout for these arguments (the
    // window's split sums follow it); the window may use fewer parts of it.
    long long stat_bytes = 0, dq_offset = 0;
    const long long need =
        bwd_ws_bytes(B, H, H_kv, T, D, head_parts(B, H, H_kv, T, D, head_split, false),
                     dq_parts_for(B, H, T, D, false), &stat_bytes, &dq_offset);
    if (need < 0) return FA_ERR_OVERFLOW;
    if (workspace_bytes < need) return FA_ERR_WORKSPACE;
    // element counts, 32-bit staging ranges (64 rows of a tile) and grids
    long long e;
    if (__builtin_mul_overflow((long long)B * T, (long long)H * D, &e) || e > kMaxElems)
        return FA_ERR_OVERFLOW;
    if ((63LL * H * D + D) * 2 >= (1LL << 31)) return FA_ERR_OVERFLOW;
    const long long nblk = ((long long)T + kBlk - 1) / kBlk;
    if ((long long)B * H * nblk > kMaxGridB || (long long)B * H_kv * nblk * hs > kMaxGridB)
        return FA_ERR_OVERFLOW;
    if ((long long)B * T * H_kv * D / 1024 + 1 > kMaxGridB)
        return FA_ERR_OVERFLOW;

    BwdParams p;
    p.q = q; p.k = k; p.v = v; p.o = o; p.dout = dout; p.lse = lse;
    p.dq = dq; p.dk = dk; p.dv = dv;
    p.delta = (float *)workspace;
    p.l2 = p.delta + (long long)B * H * T;
    p.B = B; p.H = H; p.H_kv = H_kv; p.T = T;
    p.group = H / H_kv;
    p.nblk = (int)nblk;
    p.dq_groups = dq_groups_for(B, H, T, D, window >= 0);
    p.dq_parts = dq_parts_for(B, H, T, D, window >= 0);
    p.dqpart = p.dq_parts > 1 ? (float *)((char *)workspace + dq_offset) : nullptr;
    p.c = scale * kLog2e;
    p.scale = scale;
    p.hsplit = hs;
    p.vlds = dkdv_vlds(B, H_kv, T, D, window >= 0) ? 1 : 0;
    p.klds = dkdv_klds((long long)B * H_kv * nblk * hs, D, window >= 0) ? 1 : 0;
    p.dkpart = p.dvpart = nullptr;
    if (hs > 1) {
        p.dkpart = (float *)((char *)workspace + stat_bytes);
        p.dvpart = p.dkpart + (long long)hs * B * T * H_kv * D;
    }
    p.window = window < 0 ? -1 : (window < T ? window : T);
    p.gbits = window < 0 ? nullptr : (const unsigned long long *)global_bits;
    p.nwords = (int)(((long long)T + 63) / 64);
    // Window split: as many global-key slots as the workspace holds past
    // what fa_bwd needs (none: every global tile keeps the full walk).
    p.nslots = p.nchunk = p.nfar = 0;
    p.nparts = hs;
    p.gmeta = nullptr;
    p.gpk = p.gpv = nullptr;
    if (window >= 0 && global_bits) {
        const int nch = far_chunks(T, p.window, p.group, hs);
        const int nparts = hs + nch;
        const long long avail = workspace_bytes - need;
        long long per;
        if (!__builtin_mul_overflow((long long)nparts * B, (long long)H_kv * D * 8, &per)) {
            // split_bytes(s) >= 16 + s * (per + 4): start from that bound
            long long slots = avail > 16 ? (avail - 16) / (per + 4) : 0;
            if (slots > T) slots = T;
            while (slots > 0 && split_bytes(slots, nparts, B, H_kv, D) > avail) --slots;
            const long long nfar = (long long)B * H_kv * nch;
            if (slots > 0 && (long long)B * H_kv * nblk * hs + nfar <= kMaxGridB &&
                slots * B * H_kv * (D / 4) / 256 + 1 <= kMaxGridB) {
                p.nslots = (int)slots;
                p.nchunk = nch;
                p.nparts = nparts;
                p.nfar = (int)nfar;
                char *base = (char *)workspace + need;
                p.gmeta = (int *)base;
                p.gpk = (float *)(base + 16 + (slots * 4 + 15) / 16 * 16);
                p.gpv = p.gpk + slots * nparts * B * H_kv * D;
            }
        }
    }
    hipStream_t s = (hipStream_t)stream;
    const bool win = window >= 0;
    hipError_t le;
    if (dtype == FA_DTYPE_BF16)
        le = win ? launch_bwd_c<__bf16, true>(p, D, causal, s)
                 : launch_bwd_c<__bf16, false>(p, D, causal, s);
    else
        le = win ? launch_bwd_c<_Float16, true>(p, D, causal, s)
                 : launch_bwd_c<_Float16, false>(p, D, causal, s);
    return le == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

extern "C" int fa_bwd(const void *q, const void *k, const void *v, const void *o,
                      const float *lse, const void *dout, void *dq, void *dk, void *dv, int B,
                      int H, int H_kv, int T, int D, int causal, float scale, int dtype,
                      int head_split, void *workspace, long long workspace_bytes, void *stream) {
    return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, B, H, H_kv, T, D, causal, scale, dtype,
                    -1, nullptr, head_split, workspace, workspace_bytes, stream);
}

extern "C" int fa_bwd_window(const void *q, const void *k, const void *v, const void *o,
                             const float *lse, const void *dout, void *dq, void *dk, void *dv,
                             int B, int H, int H_kv, int T, int D, int causal, float scale,
                             int dtype, int window, const void *global_bits, int head_split,
                             void *workspace, long long workspace_bytes, void *stream) {
    if (window < 0) return FA_ERR_BAD_SHAPE;
    return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, B, H, H_kv, T, D, causal, scale, dtype,
                    window, global_bits, head_split, workspace, workspace_bytes, stream);
}
