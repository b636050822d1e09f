// k3_skinny.h -- the MFMA engine for 5..64 tokens: out[t][n] = sum_k W[n][k] x[t][k].
//
// "Hyper Optimizing Kimi K3 in vLLM", Part 1 section 1 ("Tune shapes for
// the workload"): above batch 2 the projections switch to split-K kernels.
// Here a workgroup owns a tile of 16 TPW WPB weight rows (WPB waves of 16 TPW
// rows; TPW = 2 at 33-64 tokens, else 1; WPB = 4, or 6-7 for the dense
// projections at 33-64 tokens) and one of `ksplit` K ranges; its waves
// share each K chunk of the token rows, staged in LDS, while each wave
// streams its own rows with two register buffers in flight. The product
// runs on v_mfma_f32_16x16x32_bf16 with the tokens as the A operand (up to
// four 16-token tiles) and the weight rows as B. A job's epilogue either
// writes fp32 partial sums per K range (summed in a fixed order by a small
// reduce kernel), or, with one K range, finishes the outputs directly. The
// token-resident pass after it stages a whole K range once instead (dense
// projections at 5-32 tokens), and the whole-K pass at the end of the file
// gives each workgroup whole rows and no partial sums (single dense
// projections at 5-32 tokens).
#pragma once
#include "k3_device.h"

namespace k3 {

constexpr int kSkKc = 256;            // K per chunk
constexpr int kSkKb = kSkKc / 32;     // MFMA k-steps per chunk
constexpr int kSkMaxSplit = 8;        // most K ranges a projection is split into

// Weight operand loads. One load instruction covers 8 rows x 128 bytes of the
// wave's 16-row tile (h the instruction's half), so each row is fetched in
// whole 128-byte lines, in one of two lane layouts:
//   interleaved (RC = false): lane l reads row 8h + l % 8 at bytes 16 (l / 8)
//     of the piece; one DPP exchange per vector turns a pair of halves into
//     MFMA operands;
//   row-contiguous (RC = true): lane l reads row 8h + l / 8 at bytes
//     16 (l % 8), so each group of four lanes covers 64 contiguous bytes of
//     one row; the operands then also need a cross-lane permutation
//     (ds_bpermute, four per vector).
// Per load instruction the interleaved layout makes the L1 cache handle
// four times the accesses (hardware counters: 44 against 15 per
// instruction); at 33-64 tokens, where each operand feeds four MFMAs, the
// row-contiguous layout is faster (chain of projections at 64 tokens 85.0
// -> 82.1 us, 64-token Zipf MoE block 847 -> 835 us), and at 5-32 tokens the
// permutation costs more than it saves (expert stream 2-3% slower), so
// those keep the interleaved layout. (Loading the MFMA operand order
// directly, 16 rows x 64 bytes per instruction, streams about a quarter
// slower than either.) With TPW 16-row tiles per wave (the wave's 16 TPW
// contiguous rows) over a K chunk of kSkKc / TPW, load u holds tile
// u / (8 / TPW), piece (u / 2) % (4 / TPW), half u % 2. With TPW = 2 a
// staged token chunk and each token operand read from LDS serve twice the
// weight rows.
// sk_wload_p issues the loads of piece p (every tile, both halves);
// sk_wload_t the whole chunk.
template <int TPW, bool RC>
__device__ __forceinline__ void sk_wload_p(u32x4 (&buf)[kSkKb], rsrc_t rw, int c, int K, int lane,
                                           int p) {
    constexpr int KC = kSkKc / TPW, PP = KC / 64;
    const int r8 = RC ? lane >> 3 : lane & 7, q = RC ? lane & 7 : lane >> 3;
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int u = tt * 2 * PP + 2 * p + h;
            const int row = 16 * tt + 8 * h + r8;
            const int k = c * KC + 64 * p + 8 * q;
            // past K: the sign bit of K - 1 - k moves the offset out of the
            // range (reads zero); arithmetic rather than a select, which the
            // compiler would turn into a branch and a wait around the load
            const uint32_t past = (uint32_t)(K - 1 - k) & 0x80000000u;
            buf[u] = ld_weight16(rw, ((uint32_t)(row * K + k) * 2u) | past);
        }
}
template <int TPW, bool RC>
__device__ __forceinline__ void sk_wload_t(u32x4 (&buf)[kSkKb], rsrc_t rw, int c, int K,
                                           int lane) {
#pragma unroll
    for (int p = 0; p < kSkKc / TPW / 64; ++p)
        sk_wload_p<TPW, RC>(buf, rw, c, K, lane, p);
}

// The two loads of one piece (x: rows 0-7, y: rows 8-15) -> the B operands of
// its two MFMA k-steps, row l % 16 in lane l (lane group g = l / 16 holds
// eight consecutive elements of the piece).
//   interleaved: lanes l and l ^ 8 trade one vector (row_ror:8 within each
//     16-lane row, written into half the banks); step 0 then holds elements
//     16g .. 16g + 7, step 1 elements 16g + 8 .. 16g + 15;
//   row-contiguous: within each 16-lane row the lanes of quads 1 and 3 take
//     y's vector from four lanes down (p0) and those of quads 0 and 2 x's
//     from four lanes up (p1), so lane 8m + 4b + j of p0 holds row 8b + m,
//     elements 8j .. 8j + 7 (p1: 32 + 8j ..); then lane 16g + n reads lane
//     8 (n % 8) + 4 (n / 8) + g: step 0 holds elements 8g .. 8g + 7, step 1
//     elements 32 + 8g .. 32 + 8g + 7.
// sk_a_vec gives the matching token operand: the 16-byte vector of the piece
// that lane group g multiplies in step s.
template <bool RC>
__device__ __forceinline__ void sk_pair(const u32x4 &x, const u32x4 &y, u32x4 &s0, u32x4 &s1) {
    if (!RC) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s0[i] = (uint32_t)__builtin_amdgcn_update_dpp((int)x[i], (int)y[i], 0x128, 0xf, 0xc,
                                                          false);
            s1[i] = (uint32_t)__builtin_amdgcn_update_dpp((int)y[i], (int)x[i], 0x128, 0xf, 0x3,
                                                          false);
        }
        return;
    }
    const int lane = threadIdx.x & (kWave - 1), n = lane & 15;
    const int src = 4 * (8 * (n & 7) + 4 * (n >> 3) + (lane >> 4));  // byte address of the lane
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int p0 = __builtin_amdgcn_update_dpp((int)x[i], (int)y[i], 0x114, 0xf, 0xa, false);
        const int p1 = __builtin_amdgcn_update_dpp((int)y[i], (int)x[i], 0x104, 0xf, 0x5, false);
        s0[i] = (uint32_t)__builtin_amdgcn_ds_bpermute(src, p0);
        s1[i] = (uint32_t)__builtin_amdgcn_ds_bpermute(src, p1);
    }
}

template <bool RC>
__device__ __forceinline__ int sk_a_vec(int p, int g, int s) {
    return RC ? 8 * p + 4 * s + g : 8 * p + 2 * g + s;
}

// The compiler may not move instructions across this point: it keeps a
// chunk's prefetch loads ahead of the multiplies of the chunk before (left
// to itself it sinks them below, to save registers, which leaves one chunk
// in flight instead of two).
__device__ __forceinline__ void sk_keep_order() { __builtin_amdgcn_sched_barrier(0); }

// acc[tt][mt] += tokens 16 mt .. 16 mt + 15 (staged chunk xs) x tile tt of
// the wave's rows (loads buf of the same chunk). ld(p) issues piece p of the
// next chunk's weight loads just before piece p is multiplied, so a step's
// loads go out spread over its multiplies rather than in one burst ahead of
// them (chain of projections at 64 tokens 84.1 -> 83.3 us, 64-token Zipf
// MoE block 830 -> 825 us, 8-16 tokens unchanged; in-process A/B).
template <int MT, int TPW, bool RC, class Ld>
__device__ __forceinline__ void sk_mfma_chunk(f32x4 (&acc)[TPW][MT], const u32x4 (&buf)[kSkKb],
                                              const u32x4 (&xs)[MT * 16][kSkKc / TPW / 8 + 1],
                                              int mt_n, int lane, Ld ld) {
    constexpr int PP = kSkKc / TPW / 64;
    const int g = lane >> 4, rl = lane & 15;
#pragma unroll
    for (int p = 0; p < PP; ++p) {
        ld(p);
        sk_keep_order();
        u32x4 b0[TPW], b1[TPW];
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt)
            sk_pair<RC>(buf[tt * 2 * PP + 2 * p], buf[tt * 2 * PP + 2 * p + 1], b0[tt], b1[tt]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            if (mt < mt_n) {
                const u32x4 a0 = xs[mt * 16 + rl][sk_a_vec<RC>(p, g, 0)];
                const u32x4 a1 = xs[mt * 16 + rl][sk_a_vec<RC>(p, g, 1)];
#pragma unroll
                for (int tt = 0; tt < TPW; ++tt) {
                    acc[tt][mt] = mfma16x16x32(a0, b0[tt], acc[tt][mt]);
                    acc[tt][mt] = mfma16x16x32(a1, b1[tt], acc[tt][mt]);
                }
            }
        sk_keep_order();
    }
}

// Jobs policy (see SkDense and the expert jobs in experts.hip):
//   int  count()                          jobs in this launch (may read device memory)
//   int  tiles()                          tile slots per job
//   Job  job(a)                           what the item needs of job a, read once:
//                                         it has a member T (tokens; 0 skips the job)
//   void wave_rows(jb, tile, wq, w, n)    first weight row of wave wq's 16 and how many are valid
//   const uint16_t *xbase(jb)             the job's token matrix (wave-uniform)
//   int  xrow(jb, t)                      row of token t in it (t < T; may read memory)
//   int  xld(jb)                          its row stride in elements
//   void store(jb, tile, ks, wq, acc, xch)   epilogue (may hold a block barrier)
//   bool xcd_grouped()                    (stream kernel) give each XCD consecutive items
//   int  share_a(), share_p()             (stream kernel) slot shares, 0 for none (below)
// One item per loop iteration (the pipeline is filled per item): for dense
// projections, whose items are many and uniform. TPW 16-row tiles per wave
// (J.tpw must equal it) over K chunks of kSkKc / TPW: with TPW = 2 a staged
// token chunk serves twice the weight rows, which halves the token staging
// per weight byte (at 64 tokens it would otherwise equal the weight bytes).
// The K-steps run in the same order for either TPW, so the sums are the same.
// WPB waves per workgroup (J.wpb must equal it); the token buffers are the
// launch's dynamic LDS, 2 MT 16 (kSkKc / TPW / 8 + 1) 16-byte vectors.
template <int MT, class Jobs, int TPW = 1, int WPB = 4>
__global__ void __launch_bounds__(WPB * kWave) k_sk_gemm(Jobs J, int K, int ksplit) {
    constexpr int KC = kSkKc / TPW;  // K per chunk
    constexpr int KQ = KC / 8;       // 16-byte vectors per token row of a chunk
    constexpr int NT = WPB * kWave;
    // two token buffers (chunks alternate); +1 vector per row keeps the MFMA
    // reads conflict-free
    extern __shared__ u32x4 xs_lds[];
    auto &xs = *reinterpret_cast<u32x4 (*)[2][MT * 16][KQ + 1]>(xs_lds);
    __shared__ float xch[2][MT][4][kWave];  // epilogue exchange between waves
    constexpr int NV = MT * 16 * KQ;        // staged vectors per chunk
    constexpr int SQ = (NV + NT - 1) / NT;  // per thread (the last may be empty)
    static_assert(NT % KQ == 0, "each thread stages one vector column");
    const int lane = threadIdx.x & (kWave - 1), wq = wave_in_block();
    const int nchunks = (K + KC - 1) / KC;
    const int per_job = J.tiles() * ksplit;
    const int items = J.count() * per_job;
    for (int item = blockIdx.x; item < items; item += gridDim.x) {
        const int a = item / per_job, rem = item - a * per_job;
        const int tile = rem / ksplit, ks = rem - tile * ksplit;
        const auto jb = J.job(a);
        const int T = jb.T;
        if (T <= 0)
            continue;  // the whole workgroup skips together
        const int mt_n = min((T + 15) >> 4, MT);
        const uint16_t *wr;
        int nvalid;
        J.wave_rows(jb, tile, wq, wr, nvalid);
        // wave-uniform (scalar) range parts; the range itself is built where
        // it is used, so it never has to live in vector registers
        const uint16_t *wbase = uniform_ptr(wr);
        const uint32_t wbytes =
            (uint32_t)__builtin_amdgcn_readfirstlane(nvalid) * (uint32_t)K * 2u;
        // This thread stages vectors q = tid + j NT of each chunk: token
        // q / KQ, vector q % KQ. Rows past T (and vectors past NV) read zeros
        // through the buffer range (no branch, no memory access).
        const uint16_t *xb = uniform_ptr(J.xbase(jb));
        const uint32_t xld = (uint32_t)J.xld(jb);
        uint32_t xo[SQ];
        bool xv[SQ];
#pragma unroll
        for (int j = 0; j < SQ; ++j) {
            const int q = threadIdx.x + j * NT;
            const int t = q / KQ;
            xv[j] = t < T && q < NV;
            xo[j] = (uint32_t)J.xrow(jb, xv[j] ? t : 0) * xld;
        }
        const int vq = threadIdx.x % KQ;
        int c0, c1;
        split_range(nchunks, ksplit, ks, c0, c1);
        // Loads of a chunk past the item's range read nothing (an empty
        // range, offsets out of range): every load is issued on every path,
        // so the waits for a buffer count exactly the loads issued after it.
        auto wload = [&](u32x4 (&buf)[kSkKb], int c) {
            sk_wload_t<TPW, MT == 4>(buf, weight_range(wbase, c < c1 ? wbytes : 0u), c, K, lane);
        };
        auto aload = [&](u32x4 (&st)[SQ], int c) {
            const rsrc_t rx = act_range(xb);
            const int k = c * KC + 8 * vq;
            const bool kv = k < K && c < c1;
#pragma unroll
            for (int j = 0; j < SQ; ++j)
                st[j] = ld_act16(rx, (xv[j] && kv) ? (xo[j] + (uint32_t)k) * 2u : kOffNone);
        };
        auto astore = [&](u32x4 (&st)[SQ], int b) {
#pragma unroll
            for (int j = 0; j < SQ; ++j) {
                const int q = threadIdx.x + j * NT;
                if (NV % NT == 0 || q < NV)
                    xs[b][q / KQ][q % KQ] = st[j];
            }
        };
        f32x4 acc[TPW][MT];
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[tt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        // multiply chunk buffer buf (token buffer b) while chunk cn's weights
        // go out into nb
        auto compute = [&](u32x4 (&buf)[kSkKb], int b, u32x4 (&nb)[kSkKb], int cn) {
            const rsrc_t rw = weight_range(wbase, cn < c1 ? wbytes : 0u);
            sk_mfma_chunk<MT, TPW, MT == 4>(acc, buf, xs[b], mt_n, lane, [&](int p) {
                sk_wload_p<TPW, MT == 4>(nb, rw, cn, K, lane, p);
            });
        };
        // Chunk c (the item's chunks alternate between token buffers 0 and 1):
        // chunk c is multiplied while the weights of chunk c + 1 go out, the tokens
        // of chunk c + 1 (loaded one step earlier) go to the other buffer and
        // the tokens of chunk c + 2 go out; one barrier per chunk. A token
        // load thus has a whole step to arrive, and each wait is for loads
        // issued a step before. Chunks run in pairs; an odd count ends with
        // an empty chunk (zero weights and tokens, adding +0), so the loop has
        // one exit and every load is issued on every path.
        u32x4 A[kSkKb], B[kSkKb], st[SQ];
        aload(st, c0);
        wload(A, c0);
        astore(st, 0);
        aload(st, c0 + 1);
        __syncthreads();
        for (int c = c0; c < c1; c += 2) {
            compute(A, 0, B, c + 1);
            astore(st, 1);
            aload(st, c + 2);
            __syncthreads();
            compute(B, 1, A, c + 2);
            astore(st, 0);
            aload(st, c + 3);
            __syncthreads();
        }
        // acc[tt][mt][i] = out[token 16 mt + 4 g + i][row rl of the wave's tile tt]
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt)
            J.store(jb, tile, ks, wq, tt, acc[tt], xch);
        __syncthreads();  // xs and xch are reused by the next item
    }
}

// For lists of jobs (the heavy experts), whose workgroups stream several
// items each. The workgroup's units are (item, chunk) pairs: items
// blockIdx.x, blockIdx.x + gridDim.x, ... that have tokens, each over its
// chunk range. Three cursors walk that one sequence: the unit being
// multiplied, the unit whose weights are loading (one ahead) and the unit
// whose tokens are loading (two ahead), so the pipeline never drains at an
// item boundary. A step is one unit with one barrier; steps run in pairs and
// a sequence of odd length ends with an empty step (every load out of range,
// no multiply), so the loop has one exit and every load is issued on every
// path.
template <class Job>
struct SkCursor {
    int it;     // this workgroup's item index
    int c, c1;  // current chunk, end of the item's chunk range
    int tile, ks;
    Job jb;
    bool valid;
};

// TPW 16-row tiles per wave (1 or 2; J.tpw must equal it): chunks of
// kSkKc / TPW, every staged token chunk serving 64 TPW weight rows.
template <int MT, class Jobs, int TPW = 1>
__global__ void __launch_bounds__(kBlock) k_sk_gemm_stream(Jobs J, int K, int ksplit) {
    constexpr int KC = kSkKc / TPW;  // K per chunk
    constexpr int KQ = KC / 8;       // 16-byte vectors per token row of a chunk
    // two token buffers (units alternate); +1 vector per row keeps the MFMA
    // reads conflict-free
    __shared__ u32x4 xs[2][MT * 16][KQ + 1];
    __shared__ float xch[2][MT][4][kWave];  // epilogue exchange between waves
    constexpr int SQ = MT * 16 * KQ / kBlock;  // staged vectors per thread per chunk
    using Job = typename Jobs::Job;
    using Cur = SkCursor<Job>;
    const int lane = threadIdx.x & (kWave - 1), wq = wave_in_block();
    const int nchunks = (K + KC - 1) / KC;
    const int per_job = J.tiles() * ksplit;
    const int items = J.count() * per_job;
    const int vq = threadIdx.x % KQ;

    // Workgroups are dispatched to the 8 XCDs in turn, so consecutive items
    // (the tiles of one expert) normally run on 8 XCDs. Grouped, workgroup b
    // takes, in every full round of G items, the item of virtual index
    // (b % 8) G / 8 + b / 8: each XCD takes a consecutive block of the round
    // and one expert's token rows stay in one L2. A partial last round keeps
    // the plain interleave, so its items spread over every XCD. Either way
    // every item has exactly one workgroup. u.it is the round of the item.
    const int G = gridDim.x, bx = blockIdx.x;
    const int vb = (J.xcd_grouped() && G % 8 == 0) ? (bx % 8) * (G / 8) + bx / 8 : bx;
    const int nfull = items / G;
    // Slot shares (share_p > 0, set only for a grid of two workgroups per
    // compute unit): workgroups b and b + G / 2 share a compute unit, and the
    // first-dispatched one is served faster. The items then come in rounds of G / 2, item cu of a
    // round (XCD-grouped as above in full rounds) to compute unit cu, and of
    // every share_p rounds the unit's first workgroup takes the first
    // share_a, its second the others. Every item still has exactly one
    // workgroup; u.it is then the round of G / 2.
    const int sp = J.share_p(), sa = J.share_a();
    const bool shares = sp > 0 && G % 16 == 0;
    const int ncu = G / 2, slot = bx / ncu, cu = bx - slot * ncu;
    const int vcu = J.xcd_grouped() ? (cu % 8) * (ncu / 8) + cu / 8 : cu;
    const int nfullq = ncu > 0 ? items / ncu : 0;
    auto open = [&](Cur &u, int from) {
        u.valid = false;
        u.c = 0;
        u.c1 = 0;
        u.tile = 0;
        u.ks = 0;
        u.jb = Job{};
        const int rstep = shares ? ncu : (int)gridDim.x;
        for (int r = from; r * rstep < items; ++r) {
            int it;
            if (shares) {
                if ((slot == 0) != (r % sp < sa))
                    continue;  // the other workgroup's round
                it = r * ncu + (r < nfullq ? vcu : cu);
            } else {
                it = r * (int)gridDim.x + (r < nfull ? vb : (int)blockIdx.x);
            }
            if (it >= items)
                break;
            const int a = it / per_job, rem = it - a * per_job;
            const Job jb = J.job(a);
            if (jb.T <= 0)
                continue;  // uniform over the workgroup
            u.it = r;
            u.jb = jb;
            u.tile = rem / ksplit;
            u.ks = rem - u.tile * ksplit;
            split_range(nchunks, ksplit, u.ks, u.c, u.c1);
            if (u.c < u.c1) {
                u.valid = true;
                return;
            }
        }
    };
    auto next = [&](Cur &u) {
        if (u.valid && ++u.c >= u.c1)
            open(u, u.it + 1);
    };

    // token cursor: this thread stages vectors q = tid + j * 256 of each
    // chunk (token q / KQ, vector q % KQ); rows past T read zeros
    // xr holds the rows as read: they are first used by the next token load,
    // a step later, so waiting for a row lookup never waits for the weight
    // loads issued after it
    int xr[SQ];
    bool xv[SQ];
    const uint16_t *xb = nullptr;
    uint32_t xld = 0;
    auto set_rows = [&](const Cur &u) {
        xb = u.valid ? J.xbase(u.jb) : nullptr;
        xld = u.valid ? (uint32_t)J.xld(u.jb) : 0u;
#pragma unroll
        for (int j = 0; j < SQ; ++j) {
            const int t = (threadIdx.x + j * kBlock) / KQ;
            xv[j] = u.valid && t < u.jb.T;
            xr[j] = J.xrow(u.jb, xv[j] ? t : 0);  // an empty cursor has T = 0: row 0
        }
    };
    auto wload = [&](u32x4 (&buf)[kSkKb], const Cur &u) {
        const uint16_t *wr;
        int nvalid;
        J.wave_rows(u.jb, u.tile, wq, wr, nvalid);
        // range parts from lane 0: the cursor passes through joins the
        // compiler cannot prove uniform, and a range in vector registers
        // turns every load into a loop over lanes
        const uint32_t wbytes =
            u.valid ? (uint32_t)__builtin_amdgcn_readfirstlane(nvalid) * (uint32_t)K * 2u : 0u;
        sk_wload_t<TPW, MT == 4>(buf, weight_range(uniform_ptr(wr), wbytes), u.c, K, lane);
    };
    auto aload = [&](u32x4 (&st)[SQ], const Cur &u) {
        const rsrc_t rx = act_range(uniform_ptr(xb));
        const int k = u.c * KC + 8 * vq;
        const bool kv = u.valid && k < K;
#pragma unroll
        for (int j = 0; j < SQ; ++j)
            st[j] = ld_act16(rx, (xv[j] && kv) ? ((uint32_t)xr[j] * xld + (uint32_t)k) * 2u
                                               : kOffNone);
    };
    auto astore = [&](u32x4 (&st)[SQ], int b) {
#pragma unroll
        for (int j = 0; j < SQ; ++j) {
            const int q = threadIdx.x + j * kBlock;
            xs[b][q / KQ][q % KQ] = st[j];
        }
    };
    f32x4 acc[TPW][MT];
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            acc[tt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

    Cur C, W, A;  // multiply, weights (one ahead), tokens (two ahead)
    open(C, 0);
    if (!C.valid)
        return;
    W = C;
    A = C;
    u32x4 Bx[kSkKb], By[kSkKb], st[SQ];
    set_rows(A);
    aload(st, A);
    wload(Bx, W);
    astore(st, 0);
    {
        const int it0 = A.it;
        next(A);
        if (!A.valid || A.it != it0)
            set_rows(A);
    }
    aload(st, A);
    next(W);
    {
        const int it0 = A.it;
        next(A);
        if (!A.valid || A.it != it0)
            set_rows(A);
    }
    __syncthreads();

    // one unit: C multiplies from token buffer b, W's weights go out into
    // nbuf, A's tokens (already staged in st for unit C + 1) go to buffer
    // b ^ 1 and the tokens of the unit after go out
    auto step = [&](u32x4 (&buf)[kSkKb], u32x4 (&nbuf)[kSkKb], int b) {
        const uint16_t *wr;
        int nvalid;
        J.wave_rows(W.jb, W.tile, wq, wr, nvalid);
        const uint32_t wbytes =
            W.valid ? (uint32_t)__builtin_amdgcn_readfirstlane(nvalid) * (uint32_t)K * 2u : 0u;
        const rsrc_t rw = weight_range(uniform_ptr(wr), wbytes);
        const int wc = W.c;
        const int mt_n = C.valid ? min((C.jb.T + 15) >> 4, MT) : 0;
        sk_mfma_chunk<MT, TPW, MT == 4>(acc, buf, xs[b], mt_n, lane, [&](int p) {
            sk_wload_p<TPW, MT == 4>(nbuf, rw, wc, K, lane, p);
        });
        if (C.valid && C.c + 1 >= C.c1) {
            // acc[tt][mt][i] = out[token 16 mt + 4 g + i][row rl of the
            // wave's tile tt]
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt) {
                J.store(C.jb, C.tile, C.ks, wq, tt, acc[tt], xch);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    acc[tt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
        astore(st, b ^ 1);
        aload(st, A);
        next(C);
        next(W);
        const int it0 = A.it;
        const bool was = A.valid;
        next(A);
        if (was && (!A.valid || A.it != it0))
            set_rows(A);
        __syncthreads();
    };
    do {
        step(Bx, By, 0);
        step(By, Bx, 1);
    } while (C.valid);
}

// One dense projection made of up to three row segments (e.g. router,
// latent and shared gate/up rows, all against the same tokens). Segment s
// has N[s] rows (a multiple of 16) of W[s]; its rows are numbered after the
// previous segments' rows in the output. A tile is 64 tpw rows (16 tpw per
// wave). The epilogue writes fp32 partials part[(ks * T + t) * ldp + n], n
// the row in that numbering.
struct SkDense {
    const uint16_t *W[3];
    int N[3];
    int tiles_before[4];  // tiles of the segments before s; [3] = all tiles
    int rows_before[3];
    int K;
    const uint16_t *x;
    int64_t ldx;
    int T;
    float *part;
    int64_t ldp;
    int tpw;  // 16-row tiles per wave
    int wpb;  // waves per workgroup: a tile is 16 tpw wpb rows

    struct Job {
        int T;
    };
    __device__ int count() const { return 1; }
    __device__ int tiles() const { return tiles_before[3]; }
    __device__ Job job(int) const { return Job{T}; }
    __device__ int seg(int tile) const {
        return tile >= tiles_before[2] ? 2 : (tile >= tiles_before[1] ? 1 : 0);
    }
    __device__ void wave_rows(const Job &, int tile, int wq, const uint16_t *&w, int &n) const {
        const int s = seg(tile);
        const int r0 = (tile - tiles_before[s]) * 16 * wpb * tpw + wq * 16 * tpw;
        n = max(0, min(16 * tpw, N[s] - r0));
        w = W[s] + (int64_t)(n > 0 ? r0 : 0) * K;
    }
    __device__ const uint16_t *xbase(const Job &) const { return x; }
    __device__ int xrow(const Job &, int t) const { return t; }
    __device__ int xld(const Job &) const { return (int)ldx; }
    // Epilogue of tile tt of the wave's tpw tiles.
    template <int MT>
    __device__ __forceinline__ void store(const Job &, int tile, int ks, int wq, int tt,
                                          const f32x4 (&acc)[MT],
                                          float (*)[MT][4][kWave]) const {
        const int lane = threadIdx.x & (kWave - 1);
        const int s = seg(tile);
        const int r =
            (tile - tiles_before[s]) * 16 * wpb * tpw + wq * 16 * tpw + 16 * tt + (lane & 15);
        if (r >= N[s])
            return;
        const int n = rows_before[s] + r;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = mt * 16 + 4 * (lane >> 4) + i;
                if (t < T)
                    part[((int64_t)ks * T + t) * ldp + n] = acc[mt][i];
            }
    }
};

// ------------------------------------------------------------------ token-resident dense pass
// For dense projections (every row against the same tokens): workgroup b owns
// K range ks = b % ksplit, [ks kr, ks kr + kr), and stages the tokens of that
// range into LDS once; then each of its WPB waves streams its own 16-row
// tiles of the projection through the range, with two register buffers in
// flight and no barrier, from one tile to the next without draining. The
// rows are numbered over the segments of J (16-row tiles, a segment's last one
// may be partial); the workgroups of one K range take tiles wave by wave in
// turn, and the tiles of a last, partial round go to waves in an order that
// visits every compute unit before any twice (below). The epilogue writes
// each tile's fp32 partial sums for its K range
// (summed in range order by the finishing kernels), as SkDense::store does.
// K-steps within a range run in order, so the sums are a function of K, kr
// and the tokens alone.
constexpr int kResKc = 256;         // K per chunk (one register buffer: 16 rows x 512 bytes)
constexpr int kResMaxRange = 1024;  // widest K range (its tokens sit in LDS)

template <int MT, int WPB>
__global__ void __launch_bounds__(WPB * kWave) k_sk_res(SkDense J, int K, int ksplit, int kr) {
    extern __shared__ u32x4 xr[];  // [MT * 16][KQ + 1]: the range's tokens, zero past T and K
    const int lane = threadIdx.x & (kWave - 1);
    const int wq = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const int nch = (kr + kResKc - 1) / kResKc;
    const int KQ = nch * (kResKc / 8);  // staged vectors per token row
    const int ks = blockIdx.x % ksplit;
    const int k0 = ks * kr, k1 = min(K, k0 + kr);
    const int T = J.T;
    // tiles of the segments
    int st[4];
    st[0] = 0;
#pragma unroll
    for (int s = 0; s < 3; ++s)
        st[s + 1] = st[s] + (J.N[s] + 15) / 16;
    const int ntiles = st[3];
    const int nb = gridDim.x / ksplit;  // workgroups of this K range
    const int bw = blockIdx.x / ksplit;
    const int wpk = nb * WPB;           // waves of this K range
    const int w0 = bw * WPB + wq;
    // Full rounds: wave w0 takes tiles w0, w0 + wpk, ... The R tiles of the
    // partial last round go to the waves of rank < R, where rank counts the
    // range's H = nb / 2 compute units first: workgroups are dispatched to the
    // XCDs in turn and fill one slot on every compute unit before the second,
    // so with two per compute unit workgroups bw and bw + H share one. (The
    // plain order gave the o-projection's compute units 16 or 12 tiles at
    // 5-32 tokens.) Which wave takes a tile does not change its sums.
    const int nfull = ntiles / wpk, rlast = ntiles - nfull * wpk;
    const int H = nb / 2;
    const int rank = nb % 2 == 0 ? (wq * 2 + bw / H) * H + bw % H : w0;
    const int nitems = nfull + (rank < rlast ? 1 : 0);
    const int nunits = nitems * nch;
    // token staging: issued first, stored after the first weight loads
    constexpr int SMAX =  // vectors per thread
        (MT * 16 * (kResMaxRange / 8) + WPB * kWave - 1) / (WPB * kWave);
    const int nvec = MT * 16 * KQ;
    const rsrc_t rx = act_range(J.x);
    u32x4 sv[SMAX];
#pragma unroll
    for (int j = 0; j < SMAX; ++j) {
        const int i = threadIdx.x + j * WPB * kWave;
        const int t = i / KQ, v = i - t * KQ;
        const int k = k0 + 8 * v;
        const bool ok = i < nvec && t < T && k < k1;
        sv[j] = ld_act16(rx, ok ? ((uint32_t)t * (uint32_t)J.ldx + (uint32_t)k) * 2u : kOffNone);
    }
    // the unit u = (item u / nch, chunk u % nch) of this wave: its tile's rows
    auto rows_of = [&](int u, const uint16_t *&wr, int &nvalid, int &n0, int &nseg) {
        const int it = u / nch;
        const int g = it < nfull ? w0 + it * wpk : nfull * wpk + rank;  // tile
        const int s = g >= st[2] ? 2 : (g >= st[1] ? 1 : 0);
        const int r0 = (g - st[s]) * 16;
        nvalid = max(0, min(16, J.N[s] - r0));
        wr = J.W[s] + (int64_t)(nvalid > 0 ? r0 : 0) * K;
        n0 = J.rows_before[s] + r0;
        nseg = J.N[s] - r0;
    };
    auto load = [&](u32x4 (&buf)[kSkKb], int u) {
        const uint16_t *wr;
        int nvalid, n0, nseg;
        rows_of(u < nunits ? u : 0, wr, nvalid, n0, nseg);
        const uint32_t wbytes =
            u < nunits ? (uint32_t)__builtin_amdgcn_readfirstlane(nvalid) * (uint32_t)K * 2u : 0u;
        const rsrc_t rw = weight_range(uniform_ptr(wr), wbytes);
        const int cc = u - (u / nch) * nch;
        const int r8 = lane & 7, q = lane >> 3;  // the interleaved layout (see sk_wload_t)
#pragma unroll
        for (int e = 0; e < kSkKb; ++e) {
            const int row = 8 * (e & 1) + r8;
            const int k = k0 + cc * kResKc + 64 * (e >> 1) + 8 * q;
            const uint32_t past = (uint32_t)(k1 - 1 - k) & 0x80000000u;
            buf[e] = ld_weight16(rw, ((uint32_t)(row * K + k) * 2u) | past);
        }
    };
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int g4 = lane >> 4, rl = lane & 15;
    auto fin = [&](const u32x4 (&buf)[kSkKb], int u) {
        const int cc = u - (u / nch) * nch;
        const u32x4 *xb = xr + cc * (kResKc / 8);
#pragma unroll
        for (int p = 0; p < kSkKb / 2; ++p) {
            u32x4 b0, b1;
            sk_pair<false>(buf[2 * p], buf[2 * p + 1], b0, b1);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const u32x4 *xrow = xb + (mt * 16 + rl) * (KQ + 1);
                acc[mt] = mfma16x16x32(xrow[sk_a_vec<false>(p, g4, 0)], b0, acc[mt]);
                acc[mt] = mfma16x16x32(xrow[sk_a_vec<false>(p, g4, 1)], b1, acc[mt]);
            }
        }
        if (cc == nch - 1 && u < nunits) {
            // acc[mt][i] = out[token 16 mt + 4 g4 + i][row rl of the tile]
            const uint16_t *wr;
            int nvalid, n0, nseg;
            rows_of(u, wr, nvalid, n0, nseg);
            if (rl < nseg) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = mt * 16 + 4 * g4 + i;
                        if (t < T)
                            J.part[((int64_t)ks * T + t) * J.ldp + n0 + rl] = acc[mt][i];
                    }
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    };
    u32x4 A[kSkKb], B[kSkKb];
    load(A, 0);
    load(B, 1);
#pragma unroll
    for (int j = 0; j < SMAX; ++j) {
        const int i = threadIdx.x + j * WPB * kWave;
        if (i < nvec) {
            const int t = i / KQ;
            xr[t * (KQ + 1) + (i - t * KQ)] = sv[j];
        }
    }
    __syncthreads();
    // units run in pairs; an odd count ends with an empty unit (no weights,
    // no store), so the loop has one exit and every load is issued on every
    // path
    for (int u = 0; u < nunits; u += 2) {
        sk_keep_order();
        fin(A, u);
        load(A, u + 2);
        sk_keep_order();
        fin(B, u + 1);
        load(B, u + 3);
    }
}

}  // namespace k3

// ------------------------------------------------------------------ whole-K pass (5-32 tokens)
namespace k3 {

// Dense projections over at most kKwMaxTokens tokens with final outputs and
// no partial sums: workgroup g owns rows [g R, g R + R) (NT 16-row tiles,
// the last ones possibly short) over the whole K, and its NW waves split K
// into slices of kKwSlice (NW = K / kKwSlice). Wave w stages its slice of the
// tokens in its own LDS region (no other wave reads it) and streams that
// slice of every tile of the workgroup with two 8 KB register buffers in
// flight; at the end the NW slice sums of each output are added in wave
// order through LDS and written as bf16 (mode 0) or added to the residual
// (mode 1: h32 = bf16 residual + sum, residual = bf16(h32)). So an output's
// summation order is a function of K alone, and no finishing kernel follows.
// The slice is staged in PH parts, one part at a time: the whole slice up
// to 8 tokens (PH = 1), halves up to 16 (PH = 2), quarters up to 32 (PH = 4).
// A part's tokens are loaded into registers ahead of it (every part at the
// start for PH <= 2, the next one while the current one is multiplied for
// PH = 4) and written over the previous part once its chunks of every tile
// are multiplied. Each weight fragment meets TB 16-token blocks (TB = 2 above
// 16 tokens). A region holds 8 PH + 1 token rows (34 for TB = 2); the rows
// past T are zeros, which token rows of the MFMA tile past T read.
constexpr int kKwMaxTokens = 32;
constexpr int kKwSlice = 1024;  // K per wave

struct KwJob {
    const uint16_t *W;  // [N][K]
    int N, K;
    const uint16_t *x;  // [T][ldx]
    int64_t ldx;
    int T;
    int R;     // rows per workgroup (at most 16 NT)
    int mode;  // 0: y = bf16(x . W^T); 1: residual add
    uint16_t *y;  // mode 0: y [T][ldy]; mode 1: the residual [T][ldy], updated in place
    int64_t ldy;
    float *h32;  // mode 1: [T][ldy]
};

// Token rows of a wave's LDS region: the form's most tokens (8 PH, or 16 TB
// with two token blocks) plus zero rows: one, or two where that keeps each
// lane's share of a staged part a whole number of vectors.
constexpr int kw_rows(int ph, int tb) { return tb == 1 ? 8 * ph + 1 : 16 * tb + 2; }

// LDS bytes of k_sk_kw<NW, NT, PH, TB>: the token slices, later reused for the sums
constexpr size_t kw_lds_bytes(int nw, int nt, int ph, int tb) {
    const size_t tok = (size_t)nw * kw_rows(ph, tb) * (kKwSlice / ph / 8 + 1) * 16;
    const size_t red = (size_t)nw * nt * tb * 4 * kWave * 4;
    return tok > red ? tok : red;
}

template <int NW, int NT, int PH, int TB>
__global__ void __launch_bounds__(NW * kWave) k_sk_kw(KwJob J) {
    extern __shared__ u32x4 kw_lds[];
    constexpr int SL = kKwSlice / PH;  // K of the slice staged at once
    constexpr int KQ = SL / 8;         // 16-byte vectors per token row of it
    constexpr int RS = KQ + 1;         // row stride (+1 keeps the MFMA reads conflict-free)
    constexpr int ROWS = kw_rows(PH, TB);
    constexpr int NCH = SL / kSkKc;  // 256-wide chunks per staged part
    constexpr int NUP = NT * NCH;    // units (tile, chunk) per part
    constexpr int NU = PH * NUP;
    constexpr int SV = ROWS * KQ / kWave;  // staged vectors per lane per part
    constexpr int NS = PH <= 2 ? PH : 1;   // parts held in registers at once
    static_assert(ROWS * KQ % kWave == 0, "whole vectors per lane");
    static_assert(NU % 2 == 0, "units run in pairs");
    static_assert((TB == 1 ? 8 * PH : 16 * TB) < ROWS, "a zero row past the most tokens");
    const int lane = threadIdx.x & (kWave - 1), wq = wave_in_block();
    const int T = J.T, K = J.K;
    const int k0 = wq * kKwSlice;
    const int r0 = blockIdx.x * J.R;
    const int r1 = min(J.N, r0 + J.R);
    u32x4 *xw = kw_lds + wq * ROWS * RS;
    // part h's token vectors (row t < T from x, the others zeros) into set h % NS
    u32x4 sv[NS][SV];
    const rsrc_t rx = act_range(uniform_ptr(J.x));
    auto fetch = [&](int h) {
#pragma unroll
        for (int j = 0; j < SV; ++j) {
            const int q = lane + j * kWave;
            const int t = q / KQ, v = q - t * KQ;
            const int k = k0 + h * SL + 8 * v;
            sv[h % NS][j] = ld_act16(
                rx, t < T ? ((uint32_t)t * (uint32_t)J.ldx + (uint32_t)k) * 2u : kOffNone);
        }
    };
    auto stage = [&](int h) {
#pragma unroll
        for (int j = 0; j < SV; ++j) {
            const int q = lane + j * kWave;
            const int t = q / KQ;
            xw[t * RS + (q - t * KQ)] = sv[h % NS][j];
        }
    };
    // unit u: part u / NUP; within it tile (u % NUP) / NCH, chunk u % NCH
    // (tile-major, so each row's part streams in order)
    auto load = [&](u32x4 (&buf)[kSkKb], int u) {
        const int h = u / NUP, t = (u % NUP) / NCH, c = u % NCH;
        const int rt = r0 + 16 * t;
        const int nvalid = u < NU ? max(0, min(16, r1 - rt)) : 0;
        const rsrc_t rw =
            weight_range(uniform_ptr(J.W + (int64_t)(nvalid > 0 ? rt : 0) * K),
                         (uint32_t)__builtin_amdgcn_readfirstlane(nvalid) * (uint32_t)K * 2u);
        sk_wload_t<1, false>(buf, rw, (k0 + h * SL) / kSkKc + c, K, lane);
    };
    f32x4 acc[NT][TB];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
            acc[t][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int g = lane >> 4, rl = lane & 15;
    const u32x4 *xa[TB];  // this lane's token row in each 16-token block
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
        xa[tb] = xw + (16 * tb + rl < T ? 16 * tb + rl : T) * RS;
    auto compute = [&](const u32x4 (&buf)[kSkKb], int u) {
        const int t = (u % NUP) / NCH, c = u % NCH;
#pragma unroll
        for (int p = 0; p < kSkKb / 2; ++p) {
            u32x4 b0, b1;
            sk_pair<false>(buf[2 * p], buf[2 * p + 1], b0, b1);
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                const u32x4 *xc = xa[tb] + c * (kSkKc / 8);
                acc[t][tb] = mfma16x16x32(xc[sk_a_vec<false>(p, g, 0)], b0, acc[t][tb]);
                acc[t][tb] = mfma16x16x32(xc[sk_a_vec<false>(p, g, 1)], b1, acc[t][tb]);
            }
        }
    };
    // at a part boundary the previous part's multiplies are done: its region
    // takes the next part's tokens (other lanes of the wave read them, so a
    // barrier orders the writes before the reads), and with one register set
    // the part after that is fetched
    auto next_part = [&](int h) {
        stage(h);
        __syncthreads();
        if (NS == 1 && h + 1 < PH)
            fetch(h + 1);
    };
    u32x4 A[kSkKb], B[kSkKb];
#pragma unroll
    for (int h = 0; h < NS; ++h)
        fetch(h);
    load(A, 0);
    load(B, 1);
    next_part(0);
    // units in pairs; every load is issued on every path
#pragma unroll
    for (int u = 0; u < NU; u += 2) {
        if (u > 0 && u % NUP == 0)
            next_part(u / NUP);
        sk_keep_order();
        compute(A, u);
        load(A, u + 2);
        if ((u + 1) % NUP == 0)  // only with NUP odd (three tiles in quarters)
            next_part((u + 1) / NUP);
        sk_keep_order();
        compute(B, u + 1);
        load(B, u + 3);
    }
    __syncthreads();  // every wave is done with its token slice: reuse the LDS
    constexpr int NB = NT * TB;                      // 16x16 output blocks per wave
    float *red = reinterpret_cast<float *>(kw_lds);  // [NW][NB][4][64]
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                red[((wq * NB + t * TB + tb) * 4 + i) * kWave + lane] = acc[t][tb][i];
    __syncthreads();
    // acc[t][tb][i] of lane l = out[token 16 tb + 4 (l / 16) + i][row r0 + 16 t + l % 16]
    for (int e = threadIdx.x; e < NB * 4 * kWave; e += NW * kWave) {
        const int q = e / (4 * kWave), i = (e / kWave) & 3, ln = e & (kWave - 1);
        const int t = q / TB, tb = q - t * TB;
        float v = red[e];
#pragma unroll
        for (int w = 1; w < NW; ++w)
            v += red[w * NB * 4 * kWave + e];
        const int tok = 16 * tb + 4 * (ln >> 4) + i, n = r0 + 16 * t + (ln & 15);
        if (tok < T && n < r1) {
            const int64_t o = (int64_t)tok * J.ldy + n;
            if (J.mode == 0) {
                J.y[o] = f32_to_bf16(v);
            } else {
                const float h = bf16_to_f32(J.y[o]) + v;
                J.y[o] = f32_to_bf16(h);
                J.h32[o] = h;
            }
        }
    }
}

}  // namespace k3
