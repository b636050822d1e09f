// k3_skinny.h -- the MFMA engine for 5..64 tokens: out[t][n] = sum_k W[n][k] x[t][k].
//
// "Hyper Optimizing Kimi K3 in vLLM", Part 1 section 1 ("Tune shapes for
// the workload"): above batch 2 the projections switch to split-K kernels.
// Here a workgroup owns a tile of 64 weight rows (16 per wave) and one of
// `ksplit` K ranges; its four waves share each 256-wide K chunk of the
// token rows, staged in LDS, while each wave streams its own 16 rows with
// two register buffers in flight. The product runs on
// v_mfma_f32_16x16x32_bf16 with the tokens as the A operand (up to four
// 16-token tiles) and the weight rows as B. A job's epilogue either writes
// fp32 partial sums per K range (summed in a fixed order by a small reduce
// kernel), or, with one K range, finishes the outputs directly.
#pragma once
#include "k3_device.h"

namespace k3 {

constexpr int kSkRows = 64;           // weight rows per workgroup tile (16 per wave)
constexpr int kSkKc = 256;            // K per chunk
constexpr int kSkKq = kSkKc / 8;      // 16-byte vectors per token row of a chunk
constexpr int kSkKb = kSkKc / 32;     // MFMA k-steps per chunk
constexpr int kSkMaxSplit = 4;        // most K ranges a projection is split into
constexpr int kSkMaxTokens = 64;

// Weight operand loads. One load instruction covers 8 rows x 128 bytes: lane
// l reads row 8h + l % 8 (h the instruction's half of the wave's 16 rows) at
// bytes 16 (l / 8) of a 128-byte piece, so each row is fetched in whole
// 128-byte lines. (Loading the MFMA operand order directly, 16 rows x 64
// bytes per instruction, streams about a quarter slower.) Load 2p + h of a
// chunk holds piece p of the rows of half h.
__device__ __forceinline__ void sk_wload(u32x4 (&buf)[kSkKb], rsrc_t rw, int c, int K, int lane) {
    const int r8 = lane & 7, q = lane >> 3;
#pragma unroll
    for (int u = 0; u < kSkKb; ++u) {
        const int row = 8 * (u & 1) + r8;
        const int k = c * kSkKc + 64 * (u >> 1) + 8 * q;
        // past K: the sign bit of K - 1 - k moves the offset out of the range
        // (reads zero); arithmetic rather than a select, which the compiler
        // would turn into a branch and a wait around the load
        const uint32_t past = (uint32_t)(K - 1 - k) & 0x80000000u;
        buf[u] = ld_weight16(rw, ((uint32_t)(row * K + k) * 2u) | past);
    }
}

// The two loads of one piece (x: rows 0-7, y: rows 8-15) -> the B operands of
// its two MFMA k-steps, row l % 16 in lane l: lanes l and l ^ 8 trade one
// vector (row_ror:8 within each 16-lane row, written into half the banks).
// Step 0 then holds elements 16g .. 16g + 7 of the piece in lane group
// g = l / 16, step 1 elements 16g + 8 .. 16g + 15.
__device__ __forceinline__ void sk_pair(const u32x4 &x, const u32x4 &y, u32x4 &s0, u32x4 &s1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        s0[i] = (uint32_t)__builtin_amdgcn_update_dpp((int)x[i], (int)y[i], 0x128, 0xf, 0xc, false);
        s1[i] = (uint32_t)__builtin_amdgcn_update_dpp((int)y[i], (int)x[i], 0x128, 0xf, 0x3, false);
    }
}

// acc[mt] += tokens 16 mt .. 16 mt + 15 (staged chunk xs) x the wave's 16
// rows (loads buf of the same chunk).
template <int MT>
__device__ __forceinline__ void sk_mfma_chunk(f32x4 (&acc)[MT], const u32x4 (&buf)[kSkKb],
                                              const u32x4 (&xs)[MT * 16][kSkKq + 1], int mt_n,
                                              int lane) {
    const int g = lane >> 4, rl = lane & 15;
#pragma unroll
    for (int p = 0; p < kSkKb / 2; ++p) {
        u32x4 b0, b1;
        sk_pair(buf[2 * p], buf[2 * p + 1], b0, b1);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            if (mt < mt_n) {
                acc[mt] = mfma16x16x32(xs[mt * 16 + rl][8 * p + 2 * g], b0, acc[mt]);
                acc[mt] = mfma16x16x32(xs[mt * 16 + rl][8 * p + 2 * g + 1], b1, acc[mt]);
            }
    }
}

// Jobs policy (see SkDense and the expert jobs in experts.hip):
//   int  count()                          jobs in this launch (may read device memory)
//   int  tiles()                          tile slots per job
//   Job  job(a)                           what the item needs of job a, read once:
//                                         it has a member T (tokens; 0 skips the job)
//   void wave_rows(jb, tile, wq, w, n)    first weight row of wave wq's 16 and how many are valid
//   const uint16_t *xbase(jb)             the job's token matrix (wave-uniform)
//   uint32_t xrow(jb, t)                  element offset of token row t in it (t < T)
//   void store(jb, tile, ks, wq, acc, xch)   epilogue (may hold a block barrier)
// One item per loop iteration (the pipeline is filled per item): for dense
// projections, whose items are many and uniform.
template <int MT, class Jobs>
__global__ void __launch_bounds__(kBlock) k_sk_gemm(Jobs J, int K, int ksplit) {
    __shared__ u32x4 xs[MT * 16][kSkKq + 1];  // +1 vector per row keeps the MFMA reads conflict-free
    __shared__ float xch[2][MT][4][kWave];     // epilogue exchange between waves
    constexpr int SQ = MT * 16 * kSkKq / kBlock;  // staged vectors per thread per chunk
    const int lane = threadIdx.x & (kWave - 1), wq = wave_in_block();
    const int nchunks = (K + kSkKc - 1) / kSkKc;
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
        // This thread stages vectors q = tid + j * 256 of each chunk: token
        // q / kSkKq, vector q % kSkKq. Rows past T read zeros through the
        // buffer range (no branch, no memory access).
        const uint16_t *xb = uniform_ptr(J.xbase(jb));
        uint32_t xo[SQ];
        bool xv[SQ];
#pragma unroll
        for (int j = 0; j < SQ; ++j) {
            const int t = (threadIdx.x + j * kBlock) / kSkKq;
            xv[j] = t < T;
            xo[j] = J.xrow(jb, xv[j] ? t : 0);
        }
        const int vq = threadIdx.x % kSkKq;
        int c0, c1;
        split_range(nchunks, ksplit, ks, c0, c1);
        auto wload = [&](u32x4 (&buf)[kSkKb], int c) {
            sk_wload(buf, weight_range(wbase, wbytes), c, K, lane);
        };
        auto aload = [&](u32x4 (&st)[SQ], int c) {
            const rsrc_t rx = act_range(xb);
            const int k = c * kSkKc + 8 * vq;
            const bool kv = k < K;
#pragma unroll
            for (int j = 0; j < SQ; ++j)
                st[j] = ld_act16(rx, (xv[j] && kv) ? (xo[j] + (uint32_t)k) * 2u : kOffNone);
        };
        auto astore = [&](u32x4 (&st)[SQ]) {
#pragma unroll
            for (int j = 0; j < SQ; ++j) {
                const int q = threadIdx.x + j * kBlock;
                xs[q / kSkKq][q % kSkKq] = st[j];
            }
        };
        f32x4 acc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        auto compute = [&](u32x4 (&buf)[kSkKb]) { sk_mfma_chunk<MT>(acc, buf, xs, mt_n, lane); };
        // Weights of chunk c + 1 and the tokens of chunk c + 1 are in flight
        // while chunk c is multiplied; the token loads go out first, so
        // waiting for them never waits for the weights issued after them.
        u32x4 A[kSkKb], B[kSkKb], st[SQ];
        if (c0 < c1) {
            wload(A, c0);
            aload(st, c0);
            astore(st);
            __syncthreads();
            for (int c = c0; c < c1; c += 2) {
                if (c + 1 < c1) {
                    aload(st, c + 1);
                    wload(B, c + 1);
                }
                compute(A);
                __syncthreads();
                if (c + 1 >= c1)
                    break;
                astore(st);
                __syncthreads();
                if (c + 2 < c1) {
                    aload(st, c + 2);
                    wload(A, c + 2);
                }
                compute(B);
                __syncthreads();
                if (c + 2 >= c1)
                    break;
                astore(st);
                __syncthreads();
            }
        }
        // acc[mt][i] = out[token 16 mt + 4 g + i][row rl of this wave's 16]
        J.store(jb, tile, ks, wq, acc, xch);
        __syncthreads();  // xs and xch are reused by the next item
    }
}

// For lists of jobs (the heavy experts), whose workgroups stream several
// items each.
template <int MT, class Jobs>
struct SkItem {
    static constexpr int SQ = MT * 16 * kSkKq / kBlock;  // staged vectors per thread per chunk
    bool valid;
    int next;  // the next item index of this workgroup to look at
    int tile, ks, c0, c1, T, mt_n;
    typename Jobs::Job jb;
    const uint16_t *wbase;
    uint32_t wbytes;
    const uint16_t *xb;
    uint32_t xo[SQ];
    bool xv[SQ];
};

// The workgroup's items are blockIdx.x, blockIdx.x + gridDim.x, ...; their
// (item, chunk) units form one stream, so the next item's first chunk is
// already in flight while the current item finishes (a workgroup does not
// drain and refill the pipeline between tiles).
template <int MT, class Jobs>
__device__ __forceinline__ void sk_open_item(const Jobs &J, int from, int items, int per_job,
                                             int ksplit, int nchunks, int K, int wq,
                                             SkItem<MT, Jobs> &c) {
    constexpr int SQ = SkItem<MT, Jobs>::SQ;
    c.valid = false;
    for (int it = from; it < items; it += gridDim.x) {
        const int a = it / per_job, rem = it - a * per_job;
        c.jb = J.job(a);
        if (c.jb.T <= 0)
            continue;  // uniform over the workgroup
        c.next = it + gridDim.x;
        c.tile = rem / ksplit;
        c.ks = rem - c.tile * ksplit;
        c.T = c.jb.T;
        c.mt_n = min((c.T + 15) >> 4, MT);
        split_range(nchunks, ksplit, c.ks, c.c0, c.c1);
        const uint16_t *wr;
        int nvalid;
        J.wave_rows(c.jb, c.tile, wq, wr, nvalid);
        c.wbase = uniform_ptr(wr);
        c.wbytes = (uint32_t)__builtin_amdgcn_readfirstlane(nvalid) * (uint32_t)K * 2u;
        // this thread stages vectors q = tid + j * 256 of each chunk: token
        // q / kSkKq, vector q % kSkKq; rows past T read zeros
        c.xb = uniform_ptr(J.xbase(c.jb));
#pragma unroll
        for (int j = 0; j < SQ; ++j) {
            const int t = (threadIdx.x + j * kBlock) / kSkKq;
            c.xv[j] = t < c.T;
            c.xo[j] = J.xrow(c.jb, c.xv[j] ? t : 0);
        }
        c.valid = c.c0 < c.c1;
        if (c.valid)
            return;
    }
}

template <int MT, class Jobs>
__global__ void __launch_bounds__(kBlock) k_sk_gemm_stream(Jobs J, int K, int ksplit) {
    __shared__ u32x4 xs[MT * 16][kSkKq + 1];  // +1 vector per row keeps the MFMA reads conflict-free
    __shared__ float xch[2][MT][4][kWave];     // epilogue exchange between waves
    using Item = SkItem<MT, Jobs>;
    constexpr int SQ = Item::SQ;
    const int lane = threadIdx.x & (kWave - 1), wq = wave_in_block();
    const int nchunks = (K + kSkKc - 1) / kSkKc;
    const int per_job = J.tiles() * ksplit;
    const int items = J.count() * per_job;
    const int vq = threadIdx.x % kSkKq;

    auto wload = [&](u32x4 (&buf)[kSkKb], const Item &it, int c) {
        sk_wload(buf, weight_range(it.wbase, it.wbytes), c, K, lane);
    };
    auto aload = [&](u32x4 (&st)[SQ], const Item &it, int c) {
        const rsrc_t rx = act_range(it.xb);
        const int k = c * kSkKc + 8 * vq;
        const bool kv = k < K;
#pragma unroll
        for (int j = 0; j < SQ; ++j)
            st[j] = ld_act16(rx, (it.xv[j] && kv) ? (it.xo[j] + (uint32_t)k) * 2u : kOffNone);
    };
    auto astore = [&](u32x4 (&st)[SQ]) {
#pragma unroll
        for (int j = 0; j < SQ; ++j) {
            const int q = threadIdx.x + j * kBlock;
            xs[q / kSkKq][q % kSkKq] = st[j];
        }
    };
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](u32x4 (&buf)[kSkKb], int mt_n) {
        sk_mfma_chunk<MT>(acc, buf, xs, mt_n, lane);
    };

    // cur: the item being multiplied (chunk cc); nx: the item of the next
    // unit to load (chunk nc).
    Item cur, nx;
    sk_open_item<MT>(J, blockIdx.x, items, per_job, ksplit, nchunks, K, wq, cur);
    if (!cur.valid)
        return;
    nx = cur;
    int cc = cur.c0, nc = cur.c0;
    auto advance = [&]() {  // nx/nc -> the unit after it
        if (++nc >= nx.c1) {
            sk_open_item<MT>(J, nx.next, items, per_job, ksplit, nchunks, K, wq, nx);
            nc = nx.c0;
        }
    };
    // Weights of the next unit and its tokens are in flight while the current
    // unit is multiplied; the token loads go out first, so waiting for them
    // never waits for the weights issued after them.
    u32x4 A[kSkKb], B[kSkKb], st[SQ];
    wload(A, nx, nc);
    aload(st, nx, nc);
    astore(st);
    __syncthreads();
    advance();
    // one step: multiply `buf` (unit cur/cc) while the next unit loads into `nbuf`
    auto step = [&](u32x4 (&buf)[kSkKb], u32x4 (&nbuf)[kSkKb]) -> bool {
        const bool more = nx.valid;
        if (more) {
            aload(st, nx, nc);
            wload(nbuf, nx, nc);
        }
        compute(buf, cur.mt_n);
        if (cc + 1 >= cur.c1) {
            // acc[mt][i] = out[token 16 mt + 4 g + i][row rl of this wave's 16]
            J.store(cur.jb, cur.tile, cur.ks, wq, acc, xch);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        __syncthreads();  // every wave is done with xs (and xch)
        if (!more)
            return false;
        astore(st);
        __syncthreads();
        if (cc + 1 >= cur.c1) {
            cur = nx;
            cc = nc;
        } else {
            ++cc;
        }
        advance();
        return true;
    };
    while (true) {
        if (!step(A, B))
            break;
        if (!step(B, A))
            break;
    }
}

// One dense projection made of up to three row segments (e.g. router,
// latent and shared gate/up rows, all against the same tokens). Segment s
// has N[s] rows (a multiple of 16) of W[s]; its rows are numbered after the
// previous segments' rows in the output. The epilogue writes fp32 partials
// part[(ks * T + t) * ldp + n], n the row in that numbering.
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
        const int r0 = (tile - tiles_before[s]) * kSkRows + wq * 16;
        n = max(0, min(16, N[s] - r0));
        w = W[s] + (int64_t)(n > 0 ? r0 : 0) * K;
    }
    __device__ const uint16_t *xbase(const Job &) const { return x; }
    __device__ uint32_t xrow(const Job &, int t) const { return (uint32_t)((int64_t)t * ldx); }
    template <int MT>
    __device__ void store(const Job &, int tile, int ks, int wq, const f32x4 (&acc)[MT],
                          float (*)[MT][4][kWave]) const {
        const int lane = threadIdx.x & (kWave - 1);
        const int s = seg(tile);
        const int r = (tile - tiles_before[s]) * kSkRows + wq * 16 + (lane & 15);
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

}  // namespace k3
