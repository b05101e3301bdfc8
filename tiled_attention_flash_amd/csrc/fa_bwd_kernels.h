// fa_bwd_kernels.h -- the attention backward pass for gfx950 (MI355X, CDNA4):
// kernels and launcher templates, instantiated per head dim by
// fa_bwd_kernel.hip (D = 128) and fa_bwd_kernel_d64.hip (D = 64), which the
// build compiles with different scheduler flags.
//
// Method: page "TileLang 与机器学习训练：反向传播算子优化案例", section
// "算子拆分与流水线设计": a preprocess computing Delta from O and dO, then a
// main kernel in which each program holds a block of keys (K in shared
// memory), walks the query blocks, forms the scores K.q^T, and accumulates
// dV from the probabilities and dO, consuming lse and Delta.  Per query row
// i and key j (s = scale * q.k, P = exp(s - lse_i), Delta_i = O_i . dO_i):
//   dV_j += P_ij dO_i          dP_ij = dO_i . V_j
//   dS_ij = P_ij (dP_ij - Delta_i)
//   dK_j += scale dS_ij Q_i    dQ_i += scale dS_ij K_j
//
// Mapping onto CDNA4
// ------------------
// * fa_bwd_delta: one output row per 16 lanes, BSHD O and dO read once.
// * fa_bwd_dkdv (K/V-stationary, as on the page): a workgroup owns 32*W keys
//   of one (batch, K/V head), 32 per wavefront; each wavefront keeps its K
//   rows in VGPRs as MFMA B operands and reads its V rows, staged once in
//   LDS, as B operands per block (holding V in registers as well would take
//   the wavefront past 256 registers and to one wavefront per SIMD; this way
//   two workgroups share a CU: 35% faster at D = 128).  It walks the query blocks of
//   the heads that share the K/V head; a 32-row Q tile, dO tile and the rows'
//   LSE and Delta are staged in LDS for all wavefronts (direct HBM -> LDS
//   loads, double-buffered).  Per (32 queries x 32 keys):
//     S = Q.K^T and dP = dO.V^T   (v_mfma_f32_32x32x16_f16; lane = key,
//                                  registers = queries)
//     P, dS in fp32, rounded to fp16 as B operands
//     dV^T += dO^T.P, dK^T += Q^T.dS   (A operands by transpose reads)
//   so dK and dV of a key are summed over queries and query heads in
//   registers: no atomics.
// * fa_bwd_dq (Q-stationary; the page accumulates dQ with atomic adds into
//   a reordered layout, this build recomputes S and dP instead, which keeps
//   the result deterministic): like the forward kernel, 32 query rows per
//   wavefront with Q and dO in VGPRs, K/V tiles of 64 keys streamed through
//   LDS; per 32-key block S^T = K.Q^T, dP^T = V.dO^T, dS^T in fp32 with the
//   row's LSE and Delta per lane, then dQ^T += K^T.dS^T.
// * Tiles that are read both row-wise (b128) and transposed (b64_tr_b16)
//   are stored with one 16-byte-chunk XOR swizzle that keeps both patterns
//   free of bank conflicts (rt_chunk).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace bwd {


constexpr float kLog2e = 1.4426950408889634f;

// Physical 16-byte chunk of logical chunk c of row `row` for tiles read both
// ways: 16 consecutive rows at one logical chunk fall in 16 distinct bank
// groups, and so do 4 consecutive rows x 4 consecutive chunks (the block a
// half-wavefront transpose-reads).
template <int D>
__device__ __forceinline__ int rt_chunk(int row, int c)
{
    return D == 128 ? (c ^ (((row & 3) << 2) | ((row >> 2) & 3)))
                    : (c ^ ((((row >> 1) & 1) << 2) | ((row >> 2) & 3)));
}

// MFMA operand reads from an LDS tile of rows (D halves each) stored with
// rt_chunk, row 0 at `t`.  The swizzle is an XOR on the 16-byte chunk index,
// and the chunk index of k-step s (d block i) differs from that of step 0
// (block 0) only in bits the row part of the offset leaves clear, so each
// read offset is one XOR from a per-lane base.
template <int D>
struct TileRead {
    int row0;      // row read (A operand, tile rows): row lane%32, chunk 2s + half at s = 0
    int tr[2][2];  // transpose reads at d block 0: k-step cs, lower / upper 4-row group

    __device__ __forceinline__ void init()
    {
        const int lane = threadIdx.x & 63;
        const int row = lane & 31, half = lane >> 5;
        row0 = row * D + 8 * rt_chunk<D>(row, half);
        // 16-lane group gg = lane/16 (d half gg%2, row half gg/2), j = lane%16:
        // row 4*(gg/2) + j/4 (+ 16cs, + 8 for the upper group), d = 16*(gg%2) + 4*(j%4);
        // the swizzle depends on the row's bits 0..3, so each row group has its own base
        const int gg = lane >> 4, j = lane & 15;
        const int d = 16 * (gg & 1) + 4 * (j & 3);
#pragma unroll
        for (int cs = 0; cs < 2; ++cs)
#pragma unroll
            for (int up = 0; up < 2; ++up) {
                const int trow = 16 * cs + 8 * up + 4 * (gg >> 1) + (j >> 2);
                tr[cs][up] = trow * D + 8 * rt_chunk<D>(trow, d >> 3) + (d & 7);
            }
    }
    // lane holds row lane%32, d = 16s + 8*half .. +7
    __device__ __forceinline__ half8 row_frag(const _Float16 *t, int s) const
    {
        return lds_read16(t + (row0 ^ (16 * s)));
    }
    // d block i, rows of k-step cs in the accumulator's order (lane half h:
    // rows 16cs + 4h + 0..3, then 16cs + 8 + 4h + 0..3); d block i's chunks
    // differ from block 0's in the chunk bits the swizzle XORs with row bits
    // only, so its offsets are one XOR of 32i away
    __device__ __forceinline__ half8 tr_frag(const _Float16 *t, int i, int cs) const
    {
        const half4 lo = lds_read_tr(t + (tr[cs][0] ^ (32 * i)));
        const half4 hi = lds_read_tr(t + (tr[cs][1] ^ (32 * i)));
        return half8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
};

// Direct HBM -> LDS load of a tile of `kRows` rows (D halves each, row stride
// `row_stride` halves in memory) starting at row r0, split over W wavefronts;
// rows at or past n_rows load row n_rows - 1 instead (finite data whose
// contributions the caller masks).  Lane i of each load instruction fills
// LDS bytes 16i.. of a 1 KiB piece; the source chunk is chosen so that the
// data lands swizzled by rt_chunk.
template <int D, int W, int kRows>
struct TileLoad {
    static constexpr int kChunks = D / 8;
    static constexpr int kRowsPerLoad = 64 / kChunks;
    static constexpr int kLoads = kRows / kRowsPerLoad;
    static constexpr int kPerWave = kLoads / W;
    static_assert(kLoads % W == 0, "tile loads must split over the waves");

    __device__ __forceinline__ static void issue(const _Float16 *base, int64_t row_stride, int r0,
                                                 int n_rows, _Float16 *lds)
    {
        const int lane = threadIdx.x & 63;
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const int pc = lane % kChunks;
        const char *tile = (const char *)(base + (int64_t)r0 * row_stride);
#pragma unroll
        for (int n = 0; n < kPerWave; ++n) {
            const int blk = kPerWave * wave + n;
            int row = kRowsPerLoad * blk + lane / kChunks;
            const int lrow = row;  // swizzle by the row's place in the tile
            if (r0 + row > n_rows - 1) row = n_rows - 1 - r0;
            const uint32_t off = (uint32_t)(2 * ((int64_t)row * row_stride + 8 * rt_chunk<D>(lrow, pc)));
            dma16(tile, off, lds + 512 * blk);
        }
    }
};

// One 4-byte-per-lane direct HBM -> LDS load: the dword at base + off of
// lane i lands at lds + 4*i (lanes outside the exec mask write nothing).
// Like dma16, inline assembly, so the compiler does not wait for it before
// later LDS reads; the kernel waits for its loads itself.  `base` must be
// the same in every lane; it passes through readfirstlane so that it is
// held in scalar registers (the instruction's base operand) even where the
// compiler would otherwise keep the computed address in vector registers.
// A vector instruction that writes a scalar register (readfirstlane does)
// must be 5 wait states ahead of a memory instruction that reads it, and
// the compiler does not count the load inside the assembly: the s_nop 4
// supplies them (and the one wait state an M0 write needs before the load).
__device__ __forceinline__ void dma4(const char *base, uint32_t off, void *lds)
{
    const uint64_t p = (uint64_t)(uintptr_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
    const char *sbase = (const char *)(uintptr_t)(((uint64_t)hi << 32) | lo);
    const uint32_t m0 = (uint32_t)(uintptr_t)(LDS_AS void *)lds;
    __asm__ volatile("s_nop 4\n\tglobal_load_lds_dword %0, %1" : : "v"(off), "s"(sbase), "{m0}"(m0) : "memory");
}

struct BwdArgs {
    const _Float16 *q, *k, *v, *o, *dout;
    const float *lse;
    float *delta;
    _Float16 *dq, *dk, *dv;
    int Lq, Lk;         // query rows, key rows
    int past_len;       // position of query row 0 among the keys (causal only, else 0)
    int H, Hkv, groups;
    int n_blocks_item;  // key blocks (dkdv) or query blocks (dq) per (b, head)
    int n_items;
    int64_t n_rows;     // B * Lq * H (delta)
    float scale, c;     // c = scale * log2(e)
};

// ---------------------------------------------------------------- Delta

// Delta[b][h][i] = sum_d O[b,i,h,d] * dO[b,i,h,d] in fp32, one (b, i, h) row
// per 16 lanes, rows in BSHD order so that consecutive rows are contiguous.
template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256))) void fa_bwd_delta(const BwdArgs a)
{
    constexpr int kPer = D / 16;  // halves per lane
    const int64_t row = (int64_t)blockIdx.x * 16 + threadIdx.x / 16;
    const int sub = threadIdx.x % 16;
    float acc = 0.0f;
    if (row < a.n_rows) {
        const _Float16 *o = a.o + row * D + kPer * sub;
        const _Float16 *g = a.dout + row * D + kPer * sub;
        if constexpr (kPer == 8) {
            const half8 x = *(const half8 *)o, y = *(const half8 *)g;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc += (float)x[e] * (float)y[e];
        } else {
            const half4 x = *(const half4 *)o, y = *(const half4 *)g;
#pragma unroll
            for (int e = 0; e < 4; ++e) acc += (float)x[e] * (float)y[e];
        }
    }
    // sum over the 16 lanes of the row
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 16);
    if (row < a.n_rows && sub == 0) {
        const int64_t h = row % a.H, bi = row / a.H;
        const int64_t i = bi % a.Lq, b = bi / a.Lq;
        a.delta[(b * a.H + h) * a.Lq + i] = acc;
    }
}

// ---------------------------------------------------------------- dK, dV

template <int D, bool CAUSAL, int W>
struct DkDv {
    static constexpr int kSteps = D / 16;
    static constexpr int kDBlocks = D / 32;
    static constexpr int kBQ = 32;           // query rows per staged tile
    static constexpr int kTile = kBQ * D;    // halves per Q (or dO) tile
    using Load = TileLoad<D, W, kBQ>;

    struct Smem {
        _Float16 q[2][kTile];
        _Float16 g[2][kTile];  // dO
        float lse[2][kBQ];
        float delta[2][kBQ];
        _Float16 v[32 * W * D];  // the workgroup's V rows (read as B operands)
    };

    // stage query block qb of head h into buffer P
    __device__ __forceinline__ static void stage(const BwdArgs &a, int b, int h, int q0, Smem &sm, int P)
    {
        const int64_t row_stride = (int64_t)a.H * D;
        const _Float16 *qb = a.q + (int64_t)b * a.Lq * row_stride + (int64_t)h * D;
        const _Float16 *gb = a.dout + (int64_t)b * a.Lq * row_stride + (int64_t)h * D;
        Load::issue(qb, row_stride, q0, a.Lq, sm.q[P]);
        Load::issue(gb, row_stride, q0, a.Lq, sm.g[P]);
        // LSE and Delta of the 32 rows, by direct loads of lanes 0..31 of
        // wave 0 (a load into VGPRs and an LDS store would wait for the
        // tile loads just issued).  Rows past the end re-read row Lq-1; on
        // the one block per head that has such rows, wave 0 waits for its
        // loads and sets their LSE to +inf (probability 0), before the
        // barrier that precedes any read of the block.
        if (threadIdx.x < kBQ) {
            const int i = q0 + (int)threadIdx.x < a.Lq ? q0 + (int)threadIdx.x : a.Lq - 1;
            const int64_t r0 = ((int64_t)b * a.H + h) * a.Lq;  // row 0 of (b, h); 4 i < 2^32
            dma4((const char *)(a.lse + r0), (uint32_t)(4 * i), sm.lse[P]);
            dma4((const char *)(a.delta + r0), (uint32_t)(4 * i), sm.delta[P]);
            if (q0 + kBQ > a.Lq) {
                __builtin_amdgcn_s_waitcnt(0);
                if (q0 + (int)threadIdx.x >= a.Lq) sm.lse[P][threadIdx.x] = __builtin_huge_valf();
            }
        }
    }

    // P and dS of one 32 x 32 block as fp16 B operands: P = exp2(c s -
    // log2(e) LSE) for the visible (query, key) pairs -- key < Lk and,
    // causal, key <= query + past_len -- 0 elsewhere (rows past the last
    // query have LSE = +inf), and dS = P (dP - Delta).
    __device__ __forceinline__ static void probs(const floatx16 &s, const floatx16 &dp, const float *lse,
                                                 const float *delta, int q0, int key, int Lk, int past,
                                                 int half, float c, half8 (&pf)[2], half8 (&sf)[2])
    {
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            const float4v l4 = *(const float4v *)(&lse[8 * I + 4 * half]);
            const float4v d4 = *(const float4v *)(&delta[8 * I + 4 * half]);
            float pv[4], dsv[4];
#pragma unroll
            for (int J = 0; J < 4; ++J) {
                const int r = 4 * I + J;
                const int qi = q0 + 8 * I + 4 * half + J;
                float p = exp2_fast(__builtin_fmaf(s[r], c, -kLog2e * l4[J]));
                if ((CAUSAL && key > qi + past) || key >= Lk) p = 0.0f;
                pv[J] = p;
                dsv[J] = p * (dp[r] - d4[J]);
            }
            // register r -> k-step r/8, position r%8
#pragma unroll
            for (int J = 0; J < 4; J += 2) {
                const int r = 4 * I + J;
                const float2v p2 = {pv[J], pv[J + 1]};
                const float2v d2 = {dsv[J], dsv[J + 1]};
                const half2v hp = __builtin_convertvector(p2, half2v);
                const half2v hd = __builtin_convertvector(d2, half2v);
                pf[r >> 3][r & 7] = hp[0];
                pf[r >> 3][(r & 7) + 1] = hp[1];
                sf[r >> 3][r & 7] = hd[0];
                sf[r >> 3][(r & 7) + 1] = hd[1];
            }
        }
    }

    __device__ static void run(const BwdArgs &a)
    {
        __shared__ __attribute__((aligned(16))) Smem sm;
        const int lane = threadIdx.x & 63;
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const int col = lane & 31, half = lane >> 5;

        const int item = xcd_item(blockIdx.x, a.n_items);
        const int kb = item % a.n_blocks_item;
        const int rest = item / a.n_blocks_item;
        const int hk = rest % a.Hkv, b = rest / a.Hkv;
        const int Lq = a.Lq, Lk = a.Lk, past = a.past_len;
        const int k_wg = kb * 32 * W;                 // first key of the workgroup
        const int key = k_wg + 32 * wave + col;       // this lane's key
        const int64_t kv_stride = (int64_t)a.Hkv * D;

        // K rows of this wave as MFMA B operands: lane holds row `key`,
        // d = 16s + 8*half .. +7 (rows past the end: zeros); V rows of the
        // workgroup go to LDS once and are read as B operands per block
        half8 kf[kSteps];
        {
            const _Float16 *kr = a.k + ((int64_t)b * Lk + key) * kv_stride + (int64_t)hk * D;
#pragma unroll
            for (int s = 0; s < kSteps; ++s) {
                half8 x = {};
                if (key < Lk) x = *(const half8 *)(kr + 16 * s + 8 * half);
                kf[s] = x;
            }
            TileLoad<D, W, 32 * W>::issue(a.v + (int64_t)b * Lk * kv_stride + (int64_t)hk * D, kv_stride,
                                          k_wg, Lk, sm.v);
        }
        const _Float16 *vt = sm.v + 32 * wave * D;
        floatx16 dk[kDBlocks], dv[kDBlocks];
#pragma unroll
        for (int i = 0; i < kDBlocks; ++i) {
            dk[i] = floatx16{};
            dv[i] = floatx16{};
        }
        TileRead<D> tr;
        tr.init();

        // query blocks: causal -> from the block holding the first query
        // that sees the workgroup's first key, row k_wg - past_len (earlier
        // queries see none of its keys)
        const int n_qb = (Lq + kBQ - 1) / kBQ;
        int qb0 = 0;
        if (CAUSAL) {
            const int64_t first = (int64_t)k_wg - past;
            qb0 = first <= 0 ? 0 : (first >= (int64_t)n_qb * kBQ ? n_qb : (int)(first / kBQ));
        }
        const int per_head = n_qb - qb0;
        const int total = per_head * a.groups;
        const float c = a.c;

        if (total > 0) {
            stage(a, b, hk * a.groups, qb0 * kBQ, sm, 0);
            for (int t = 0; t < total; ++t) {
                const int P = t & 1;
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
                if (t + 1 < total) {
                    const int tn = t + 1;
                    stage(a, b, hk * a.groups + tn / per_head, (qb0 + tn % per_head) * kBQ, sm, P ^ 1);
                }
                const int q0 = (qb0 + t % per_head) * kBQ;
                const _Float16 *qt = sm.q[P], *gt = sm.g[P];

                // S = Q.K^T and dP = dO.V^T, lane = key, register r = query
                // 8(r/4) + 4*half + r%4 of the block
                floatx16 s = {}, dp = {};
#pragma unroll
                for (int st = 0; st < kSteps; ++st) {
                    s = __builtin_amdgcn_mfma_f32_32x32x16_f16(tr.row_frag(qt, st), kf[st], s, 0, 0, 0);
                    dp = __builtin_amdgcn_mfma_f32_32x32x16_f16(tr.row_frag(gt, st), tr.row_frag(vt, st), dp, 0, 0, 0);
                }
                half8 pf[2], sf[2];
                probs(s, dp, sm.lse[P], sm.delta[P], q0, key, Lk, past, half, c, pf, sf);
                // dV^T += dO^T.P, dK^T += Q^T.dS (A operands transposed)
#pragma unroll
                for (int cs = 0; cs < 2; ++cs)
#pragma unroll
                    for (int i = 0; i < kDBlocks; ++i) {
                        dv[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(tr.tr_frag(gt, i, cs), pf[cs], dv[i], 0, 0, 0);
                        dk[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(tr.tr_frag(qt, i, cs), sf[cs], dk[i], 0, 0, 0);
                    }
            }
        }

        // dK = scale dK^T^T, dV = dV^T^T: lane holds key `key`, d = 32i +
        // 8(r/4) + 4*half + r%4
        if (key < Lk) {
            _Float16 *dkr = a.dk + ((int64_t)b * Lk + key) * kv_stride + (int64_t)hk * D;
            _Float16 *dvr = a.dv + ((int64_t)b * Lk + key) * kv_stride + (int64_t)hk * D;
#pragma unroll
            for (int i = 0; i < kDBlocks; ++i)
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    const float4v k4 = {dk[i][4 * rb] * a.scale, dk[i][4 * rb + 1] * a.scale,
                                        dk[i][4 * rb + 2] * a.scale, dk[i][4 * rb + 3] * a.scale};
                    const float4v v4 = {dv[i][4 * rb], dv[i][4 * rb + 1], dv[i][4 * rb + 2], dv[i][4 * rb + 3]};
                    *(half4 *)(dkr + 32 * i + 8 * rb + 4 * half) = __builtin_convertvector(k4, half4);
                    *(half4 *)(dvr + 32 * i + 8 * rb + 4 * half) = __builtin_convertvector(v4, half4);
                }
        }
    }
};

template <int D, bool CAUSAL, int W>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * W, 64 * W), amdgpu_waves_per_eu(2, 2))) void
fa_bwd_dkdv(const BwdArgs a)
{
    DkDv<D, CAUSAL, W>::run(a);
}

// ---------------------------------------------------------------- dQ

template <int D, bool CAUSAL, int W>
struct Dq {
    static constexpr int kSteps = D / 16;
    static constexpr int kDBlocks = D / 32;
    static constexpr int kBN = 64;          // keys per staged tile
    static constexpr int kTile = kBN * D;
    static constexpr int kBM = 32 * W;      // query rows per work item
    using Load = TileLoad<D, W, kBN>;

    __device__ static void run(const BwdArgs &a)
    {
        __shared__ __attribute__((aligned(16))) _Float16 klds[2][kTile];
        __shared__ __attribute__((aligned(16))) _Float16 vlds[2][kTile];
        const int lane = threadIdx.x & 63;
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const int col = lane & 31, half = lane >> 5;

        const int item = xcd_item(blockIdx.x, a.n_items);
        int qb = item % a.n_blocks_item;
        if (CAUSAL) qb = a.n_blocks_item - 1 - qb;  // heaviest first
        const int rest = item / a.n_blocks_item;
        const int g = rest % a.groups;
        const int rest2 = rest / a.groups;
        const int hk = rest2 % a.Hkv, b = rest2 / a.Hkv;
        const int h = hk * a.groups + g;
        const int Lq = a.Lq, Lk = a.Lk, past = a.past_len;
        const int q0 = qb * kBM;
        const int qi = q0 + 32 * wave + col;  // this lane's query row
        const int64_t q_stride = (int64_t)a.H * D, kv_stride = (int64_t)a.Hkv * D;

        // Q and dO of this lane's row as MFMA B operands (rows past the end: zeros)
        half8 qf[kSteps], gf[kSteps];
        {
            const _Float16 *qr = a.q + ((int64_t)b * Lq + qi) * q_stride + (int64_t)h * D;
            const _Float16 *gr = a.dout + ((int64_t)b * Lq + qi) * q_stride + (int64_t)h * D;
#pragma unroll
            for (int s = 0; s < kSteps; ++s) {
                half8 x = {}, y = {};
                if (qi < Lq) {
                    x = *(const half8 *)(qr + 16 * s + 8 * half);
                    y = *(const half8 *)(gr + 16 * s + 8 * half);
                }
                qf[s] = x;
                gf[s] = y;
            }
        }
        const int64_t srow = ((int64_t)b * a.H + h) * Lq + qi;
        // rows past the end: LSE = +inf (probability 0), Delta = 0; a row
        // that sees no key (LSE = -inf) has every key masked below
        const float nl = qi < Lq ? -kLog2e * a.lse[srow] : -__builtin_huge_valf();
        const float dlt = qi < Lq ? a.delta[srow] : 0.0f;
        const float c = a.c;

        floatx16 dq[kDBlocks];
#pragma unroll
        for (int i = 0; i < kDBlocks; ++i) dq[i] = floatx16{};
        TileRead<D> tr;
        tr.init();

        // keys the work item can see: all Lk, or (causal) up to the position
        // of its last query row
        int kv_end = Lk;
        if (CAUSAL) {
            const int64_t last = (int64_t)(q0 + kBM < Lq ? q0 + kBM : Lq) - 1 + past;
            kv_end = last < 0 ? 0 : (last < Lk - 1 ? (int)last + 1 : Lk);
        }
        const int n_tiles = (kv_end + kBN - 1) / kBN;
        if (n_tiles > 0) {
            Load::issue(a.k + (int64_t)b * Lk * kv_stride + (int64_t)hk * D, kv_stride, 0, Lk, klds[0]);
            Load::issue(a.v + (int64_t)b * Lk * kv_stride + (int64_t)hk * D, kv_stride, 0, Lk, vlds[0]);
        }
        for (int t = 0; t < n_tiles; ++t) {
            const int P = t & 1;
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (t + 1 < n_tiles) {
                Load::issue(a.k + (int64_t)b * Lk * kv_stride + (int64_t)hk * D, kv_stride, kBN * (t + 1), Lk, klds[P ^ 1]);
                Load::issue(a.v + (int64_t)b * Lk * kv_stride + (int64_t)hk * D, kv_stride, kBN * (t + 1), Lk, vlds[P ^ 1]);
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int k0 = kBN * t + 32 * u;
                if (k0 >= kv_end) break;
                const _Float16 *kt = klds[P] + 32 * u * D, *vt = vlds[P] + 32 * u * D;
                // S^T = K.Q^T, dP^T = V.dO^T: lane = query, register r = key
                // k0 + 8(r/4) + 4*half + r%4
                floatx16 s = {}, dp = {};
#pragma unroll
                for (int st = 0; st < kSteps; ++st) {
                    s = __builtin_amdgcn_mfma_f32_32x32x16_f16(tr.row_frag(kt, st), qf[st], s, 0, 0, 0);
                    dp = __builtin_amdgcn_mfma_f32_32x32x16_f16(tr.row_frag(vt, st), gf[st], dp, 0, 0, 0);
                }
                half8 sf[2];
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    float d2[2];
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const int kj = k0 + 8 * ((r + e) >> 2) + 4 * half + ((r + e) & 3);
                        float p = exp2_fast(__builtin_fmaf(s[r + e], c, nl));
                        if ((CAUSAL && kj > qi + past) || kj >= Lk) p = 0.0f;
                        d2[e] = p * (dp[r + e] - dlt);
                    }
                    const float2v f2 = {d2[0], d2[1]};
                    const half2v h2 = __builtin_convertvector(f2, half2v);
                    sf[r >> 3][r & 7] = h2[0];
                    sf[r >> 3][(r & 7) + 1] = h2[1];
                }
                // dQ^T += K^T.dS^T
#pragma unroll
                for (int cs = 0; cs < 2; ++cs)
#pragma unroll
                    for (int i = 0; i < kDBlocks; ++i)
                        dq[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(tr.tr_frag(kt, i, cs), sf[cs], dq[i], 0, 0, 0);
            }
        }

        // dQ = scale (dQ^T)^T: lane holds row qi, d = 32i + 8(r/4) + 4*half + r%4
        if (qi < Lq) {
            _Float16 *dqr = a.dq + ((int64_t)b * Lq + qi) * q_stride + (int64_t)h * D;
#pragma unroll
            for (int i = 0; i < kDBlocks; ++i)
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    const float4v q4 = {dq[i][4 * rb] * a.scale, dq[i][4 * rb + 1] * a.scale,
                                        dq[i][4 * rb + 2] * a.scale, dq[i][4 * rb + 3] * a.scale};
                    *(half4 *)(dqr + 32 * i + 8 * rb + 4 * half) = __builtin_convertvector(q4, half4);
                }
        }
    }
};

template <int D, bool CAUSAL, int W>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * W, 64 * W), amdgpu_waves_per_eu(2, 2))) void
fa_bwd_dq(const BwdArgs a)
{
    Dq<D, CAUSAL, W>::run(a);
}

template <int D, bool CAUSAL>
int launch_bwd(BwdArgs a, int B, hipStream_t stream)
{
    // Delta
    {
        const int64_t blocks = (a.n_rows + 15) / 16;
        if (blocks > 0x7fffffff) return FA_ERR_SHAPE;
        if (blocks > 0) {
            hipLaunchKernelGGL((fa_bwd_delta<D>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
            if (hipGetLastError() != hipSuccess) return FA_ERR_LAUNCH;
        }
    }
    // dK, dV
    {
        // eight wavefronts (256 keys per workgroup, one per CU) for the full
        // pass at D = 128, four otherwise (measured per workload)
        constexpr int W = (D == 128 && !CAUSAL) ? 8 : 4;
        BwdArgs b = a;
        b.n_blocks_item = (a.Lk + 32 * W - 1) / (32 * W);
        const int64_t items = (int64_t)B * a.Hkv * b.n_blocks_item;
        if (items > 0x7fffffff) return FA_ERR_SHAPE;
        b.n_items = (int)items;
        if (items > 0) {  // none without keys
            hipLaunchKernelGGL((fa_bwd_dkdv<D, CAUSAL, W>), dim3(b.n_items), dim3(64 * W), 0, stream, b);
            if (hipGetLastError() != hipSuccess) return FA_ERR_LAUNCH;
        }
    }
    // dQ
    {
        constexpr int W = (CAUSAL || D == 64) ? 4 : 8;
        BwdArgs b = a;
        b.n_blocks_item = (a.Lq + 32 * W - 1) / (32 * W);
        const int64_t items = (int64_t)B * a.H * b.n_blocks_item;
        if (items > 0x7fffffff) return FA_ERR_SHAPE;
        b.n_items = (int)items;
        if (items > 0) {  // none without queries
            hipLaunchKernelGGL((fa_bwd_dq<D, CAUSAL, W>), dim3(b.n_items), dim3(64 * W), 0, stream, b);
            if (hipGetLastError() != hipSuccess) return FA_ERR_LAUNCH;
        }
    }
    return FA_OK;
}

// The D = 64 instances, compiled in their own translation unit.
int launch_backward_d64(const BwdArgs &a, int B, bool causal, hipStream_t stream);

}  // namespace bwd
}  // namespace fa
