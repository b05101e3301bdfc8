// fa_fwd_kernel.hip -- attention forward kernels for gfx950 (MI355X, CDNA4).
//
// Method: page "使用 TileLang 在 AMD GPU 上快速开发高性能 Flash Attention",
// sections "Q Tile 处理与缓存初始化" (one Q block per work item, fp32
// accumulator and running row max / row sum), "K/V Tile 遍历与核心计算" (K/V
// tiles streamed in order; causal loop bound; mask; Q K^T; max, rescale, exp,
// row sum; P cast to fp16; P V) and "最终输出写回与Q tile 迭代" (divide by the
// row sum with a guard, write O).  The per-row log-sum-exp that the backward
// pass consumes (page "TileLang 与机器学习训练：反向传播算子优化案例") is
// written as well.
//
// Mapping onto CDNA4
// ------------------
// * Workgroup = W wavefronts owning one block of BM = 32*W query rows of one
//   (batch, query head); each wavefront owns 32 whole query rows.  W = 8 for
//   the full (non-causal) pass at D = 128 -- each K/V tile brought into LDS
//   then serves 256 queries -- and W = 4 under the causal mask, where the
//   smaller block keeps the wavefronts of a workgroup evenly loaded along the
//   diagonal (W = 8 again from 4096 keys on, where the diagonal is a small
//   share of each work item), and at D = 64, where the shorter tiles favour
//   independent workgroups: three per CU (three wavefronts per SIMD).
// * Both products are computed transposed, on v_mfma_f32_32x32x16_f16:
//     S^T[key][query]  = K . Q^T     (A = K rows from LDS, B = Q in VGPRs)
//     O^T[d][query]   += V^T . P^T   (A = V^T from LDS,   B = P in VGPRs)
//   In the 32x32 accumulator layout lane l holds column l%32 -- one query --
//   and 16 of its 32 rows (keys, or d); the other 16 live in lane l^32.  Row
//   statistics are per-lane values plus ONE exchange between the two 32-lane
//   halves (v_permlane32_swap), and the per-row rescale of O^T is a per-lane
//   scalar.
// * The S^T accumulators, converted to fp16, are the B operand of the second
//   product once the 16 keys of each k-step are taken in the order the
//   accumulator holds them (lane half h: keys 4h..4h+3, then 8+4h..8+4h+3).
//   V stays row-major in LDS and ds_read_b64_tr_b16 (which hands lane i of a
//   16-lane group column i of the 4x16 block its group points at) builds the
//   V^T operand in exactly that key order, so P never leaves registers.
// * K/V tiles of BN = 64 keys travel HBM -> LDS with global_load_lds_dwordx4
//   (16 bytes per lane, no staging registers), double-buffered with one
//   workgroup barrier per tile; the next tile's loads fly while the current
//   one is computed.  K tiles start 32 keys after V tiles, so that the two
//   S products a tile's step issues (see below) read the K tile paired with
//   the V tile.  The source address of each lane is chosen so that rows
//   land with a 16-byte-chunk XOR swizzle that makes the K reads
//   (ds_read_b128, 16 rows per LDS cycle) and the V transpose reads (4 rows x
//   64 bytes per half-wavefront) free of bank conflicts.  Rows past the end
//   of the sequence load row L-1 instead (finite data that the mask hides).
// * Software pipeline over score blocks of 32 keys: while the matrix unit
//   computes S of block u+1, the vector ALU exponentiates block u; P.V of
//   block u follows.  The wavefront holds a raised issue priority through
//   the exponential phase, so the other wavefront of its SIMD tends to run
//   its P.V MFMAs meanwhile.
// * Online softmax against a reference maximum: block 0 sets each row's
//   reference to its exact maximum (a row that sees any key sees key 0).
//   Later blocks are exponentiated against the current reference with no
//   row maximum of their own; a block whose probabilities sum to 2^15 or
//   more in some lane (fp32 sums, so an overflow is caught too) is
//   recomputed after the reference is raised to the block's maximum and
//   O, l are rescaled.
//   Kept probabilities stay below 2^15, relative to a weight of 1 that the
//   row already holds, and the final O / l and LSE are unchanged.
// * Causal: tiles past the work item's last query are never visited; the
//   mask code runs only on blocks that straddle a wavefront's diagonal (or
//   hold the ragged end of the sequence).  A tile whose keys all lie past a
//   wavefront's last row is skipped by that wavefront, which still issues its
//   share of the loads and meets the barriers; blocks past its diagonal inside
//   a tile it does compute are computed fully masked (weights 0).
// * Output: O is normalised, rounded to fp16 and exchanged between the two
//   lane halves so that each lane stores 16 contiguous bytes of its row.
// * Grid, full pass: one workgroup per (b, kv head, group member, q block)
//   work item; workgroup ids are remapped so that each of the 8 XCDs (which
//   receive workgroups round-robin) walks a contiguous range of work items,
//   keeping one head's K/V in that XCD's L2.
// * Grid, causal: persistent, as the pages' kernel loops over q blocks -- the
//   resident workgroups walk their XCD's range of row groups in phases of a
//   few row groups, taking single q blocks heaviest first in rounds of
//   alternating direction, so that the work per workgroup evens out and no
//   workgroup is left with only diagonal-heavy blocks (see run()).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <numeric>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kBN = 64;  // keys per K/V tile in LDS

struct Args {
    const _Float16 *q, *k, *v;
    _Float16 *o;
    float *lse;
    int Lq, Lk;    // query rows, key rows
    int past_len;  // position of query row 0 among the keys (causal mask only)
    int H, Hkv, groups, n_qblocks, n_items;
    int n_rows;      // causal (persistent grid): row groups, B * H
    int phase_rows;  // causal: row groups per phase (see run())
    float scale;       // multiplier of Q.K
    float scale_log2;  // scale * log2(e): exp(scale*x) == exp2(scale_log2*x)
};

// Tile geometry for head dim D and W wavefronts.  A tile row is D halves =
// D/8 chunks of 16 bytes; one wave-wide direct load fills 1 KiB of LDS.
template <int D, int W>
struct Geo {
    static constexpr int kChunks = D / 8;              // 16-byte chunks per row
    static constexpr int kRowsPerLoad = 64 / kChunks;  // rows one wave load instruction fills
    static constexpr int kLoadsPerTile = kBN / kRowsPerLoad;
    static constexpr int kLoadsPerWave = kLoadsPerTile / W;
    static constexpr int kTile = kBN * D;  // halves per K (or V) tile
    static_assert(kLoadsPerTile % W == 0, "tile loads must split over the waves");
};

// Tile row that the n-th direct load of thread tid (lane tid%64 of wave
// tid/64) fills.
template <int D, int W>
__device__ __forceinline__ int load_row(int tid, int n)
{
    using G = Geo<D, W>;
    const int lane = tid & 63, wave = tid >> 6;
    return G::kRowsPerLoad * (G::kLoadsPerWave * wave + n) + lane / G::kChunks;
}

// Byte offsets, relative to the first key row of a tile, of the 16-byte
// chunks this lane copies with each of its direct loads.  Rows of a tile are
// < 64 apart, so the offsets fit 32 bits (the host checks Hkv*D).
template <int D, int W>
struct LoadOffsets {
    uint32_t k[Geo<D, W>::kLoadsPerWave], v[Geo<D, W>::kLoadsPerWave];
};

template <int D, int W>
__device__ __forceinline__ void init_load_offsets(LoadOffsets<D, W> &lo, int64_t kv_row, int tid)
{
    using G = Geo<D, W>;
    const int pc = (tid & 63) % G::kChunks;
#pragma unroll
    for (int n = 0; n < G::kLoadsPerWave; ++n) {
        const int row = load_row<D, W>(tid, n);
        lo.k[n] = (uint32_t)(2 * (row * kv_row + 8 * k_chunk<D>(row, pc)));
        lo.v[n] = (uint32_t)(2 * (row * kv_row + 8 * v_chunk<D>(row, pc)));
    }
}

// Issue this wave's share of the direct loads of the K (or V) tile that
// starts at key k0, whose key row 0 is at `tile` (k0 * kv_row elements past
// the head's key 0).  EDGE: the tile may start before key 0 or reach past
// Lk.  Then a row past the end re-reads row Lk-1 (finite data that the mask
// hides), and an instruction whose rows all lie before key 0 (the first K
// tile starts at key -32) is not issued -- those rows are never read.  A
// tile with every row inside [0, Lk) takes the lane offsets as they are.
template <int D, int W, bool IS_V, bool EDGE>
__device__ __forceinline__ void issue_loads(const LoadOffsets<D, W> &lo, const char *tile, int64_t kv_row,
                                            int k0, int Lk, _Float16 *lds, int wave, int tid)
{
    using G = Geo<D, W>;
#pragma unroll
    for (int n = 0; n < G::kLoadsPerWave; ++n) {
        const int blk = G::kLoadsPerWave * wave + n;
        uint32_t off = IS_V ? lo.v[n] : lo.k[n];
        if constexpr (EDGE) {
            if (k0 + G::kRowsPerLoad * blk < 0) continue;  // whole instruction before key 0
            const int over = k0 + load_row<D, W>(tid, n) - (Lk - 1);
            if (over > 0) off -= (uint32_t)(2 * over * kv_row);
        }
        dma16(tile, off, lds + 512 * blk);
    }
}

template <int D, bool CAUSAL, int W>
struct Kernel : WaveMath<D, CAUSAL> {
    using M = WaveMath<D, CAUSAL>;
    using typename M::State;
    using M::kSteps;
    using M::kDBlocks;
    using M::kCS;
    using M::kPairs;
    using M::kfrag;
    using M::vfrag;
    using M::mask;
    using M::block_max;
    using M::s_product;
    using M::rescale;
    using M::raise_to;
    using M::exp_pair;
    using G = Geo<D, W>;
    static constexpr int kThreads = 64 * W;
    static constexpr bool kPersistent = CAUSAL;  // see run()
    static constexpr int kBM = 32 * W;  // query rows per work item

    // The probabilities of a block overran the limit: raise the reference
    // maximum to the block's own (rescaling O and l) and compute them again.
    __device__ __forceinline__ static void fixup(State &st, const floatx16 &sc, half8 (&pf)[kCS],
                                                           float (&rs)[2], float c)
    {
        raise_to(st, block_max(sc), c);
        rs[0] = 0.0f;
        rs[1] = 0.0f;
#pragma unroll
        for (int p = 0; p < kPairs; ++p) exp_pair(sc, pf, rs, p, st.mc, c);
    }

    // One pipelined step for score block u, whose scores sc are complete.
    // MASK: mask sc first (the block holds keys past the end, or, causal,
    // keys after some row's position).  NEXT: the S product of block u+1
    // (into sn) is issued with the exponentials of block u between its
    // MFMAs, so the matrix unit always has work that does not wait on the
    // vector ALU.  The probabilities are taken against the current reference
    // maximum with no row maximum of their own; one wavefront-wide test of
    // the lanes' block sums sends the rare block that overruns the limit to
    // `fixup` before any of it reaches O.  Then the P.V product of block u.
    // kl: first K row of block u+1, vl: first V row of block u.
    template <bool NEXT, bool MASK>
    __device__ __forceinline__ static void step(State &st, floatx16 &sc, floatx16 &sn,
                                                const _Float16 *kl, const _Float16 *vl, int k0,
                                                int Lk, int qp, int h4, float c)
    {
        if constexpr (MASK) mask(sc, k0, Lk, qp, h4);
        // The two wavefronts that share a SIMD run best in opposite phases:
        // one exponentiating (vector ALU and matrix unit) while the other
        // feeds the matrix unit with its P.V products.  A wavefront raises
        // its issue priority for the S/exp phase and drops it for P.V, which
        // pushes the pair towards that arrangement (measured: 3% faster at
        // D = 128, 8 wavefronts).
        __builtin_amdgcn_s_setprio(1);
        half8 pf[kCS];
        float rs[2] = {0.0f, 0.0f};
        const float mc = st.mc;
        constexpr int kN = kDBlocks * kCS;
        constexpr int kVAhead = 2;  // measured about 1 % faster than 4
        half8 va[kN];

        if constexpr (NEXT) {
            constexpr int kAhead = kSteps < 4 ? kSteps : 4;
            half8 ka[kSteps];
#pragma unroll
            for (int s = 0; s < kAhead; ++s) ka[s] = kfrag(st, kl, s);
            sn = floatx16{};
#pragma unroll
            for (int s = 0; s < kSteps; ++s) {
                if (s + kAhead < kSteps) ka[s + kAhead] = kfrag(st, kl, s + kAhead);
                sn = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[s], st.qf[s], sn, 0, 0, 0);
#pragma unroll
                for (int p = kPairs * s / kSteps; p < kPairs * (s + 1) / kSteps; ++p)
                    exp_pair(sc, pf, rs, p, mc, c);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
#pragma unroll
            for (int p = 0; p < kPairs; ++p) exp_pair(sc, pf, rs, p, mc, c);
        }
        // V operands of the first P.V MFMAs in flight during the test
#pragma unroll
        for (int n = 0; n < kVAhead; ++n) va[n] = vfrag(st, vl, n % kDBlocks, n / kDBlocks);
        if (__builtin_amdgcn_ballot_w64(rs[0] + rs[1] >= kSumLimit)) fixup(st, sc, pf, rs, c);
        st.l += rs[0] + rs[1];

        __builtin_amdgcn_s_setprio(0);
        // O^T += V^T . P^T, V operands kVAhead MFMAs ahead
#pragma unroll
        for (int n = 0; n < kN; ++n) {
            if (n + kVAhead < kN) va[n + kVAhead] = vfrag(st, vl, (n + kVAhead) % kDBlocks, (n + kVAhead) / kDBlocks);
            st.oacc[n % kDBlocks] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[n], pf[n / kDBlocks],
                                                                            st.oacc[n % kDBlocks], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // LDS tile t (P = t % 2) covers score blocks u = 2t (scores in sa) and
    // 2t+1 (scores in sb).  V tile t holds keys 64t..64t+63 in vlds[t % 2];
    // K tile t holds keys 64t+32..64t+95 in klds[(t+1) % 2] -- 32 keys ahead,
    // so the two S products of the tile (blocks 2t+1 and 2t+2) read the one
    // K tile that the P.V products' V tile is paired with.  At the barrier
    // K(t) and V(t) have landed and every wavefront is done with K(t-1) and
    // V(t-1), whose buffers then receive K(t+1) and V(t+1).
    struct Ring {
        const LoadOffsets<D, W> *lo;
        const char *k0tile, *v0tile;  // K tile 0 (keys 32..95), V tile 0 (keys 0..63)
        uint32_t tile_stride;         // bytes between consecutive tiles' first key rows
        int64_t kv_row;
        int n_tiles, n_blocks, Lk, qp;
        int h4;  // 4 * (lane / 32): key offset of the lane's half in a score block
        int tid, wave;
        float c;
        _Float16 (*klds)[G::kTile];
        _Float16 (*vlds)[G::kTile];
        int wlast;  // causal: key position of the wavefront's last query row
    };

    __device__ __forceinline__ static void tile_wait()
    {
        __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of K(t), V(t) have landed
        __syncthreads();                // ... and every wave's
    }

    template <int P>
    __device__ __forceinline__ static void tile_start(const Ring &r, int t)
    {
        tile_wait();
        const int64_t step = (int64_t)(t + 1) * r.tile_stride;
        if (2 * t + 3 < r.n_blocks) {
            const int k0 = kBN * (t + 1) + kSB;
            if (k0 + kBN <= r.Lk)
                issue_loads<D, W, false, false>(*r.lo, r.k0tile + step, r.kv_row, k0, r.Lk, r.klds[P], r.wave, r.tid);
            else
                issue_loads<D, W, false, true>(*r.lo, r.k0tile + step, r.kv_row, k0, r.Lk, r.klds[P], r.wave, r.tid);
        }
        if (t + 1 < r.n_tiles) {
            const int v0 = kBN * (t + 1);
            if (v0 + kBN <= r.Lk)
                issue_loads<D, W, true, false>(*r.lo, r.v0tile + step, r.kv_row, v0, r.Lk, r.vlds[P ^ 1], r.wave, r.tid);
            else
                issue_loads<D, W, true, true>(*r.lo, r.v0tile + step, r.kv_row, v0, r.Lk, r.vlds[P ^ 1], r.wave, r.tid);
        }
    }

    // a tile whose two blocks both have a successor; MASK: mask both blocks
    template <int P, bool MASK>
    __device__ __forceinline__ static void tile(State &st, floatx16 &sa, floatx16 &sb, const Ring &r, int t)
    {
        tile_start<P>(r, t);
        // causal: every key of this and of every later tile lies past the
        // wavefront's last row, so their weights are all 0 -- the wavefront
        // only keeps loading and meeting the barriers
        if (CAUSAL && MASK && kBN * t > r.wlast) return;
        const _Float16 *kl = r.klds[P ^ 1], *vl = r.vlds[P];
        step<true, MASK>(st, sa, sb, kl, vl, kBN * t, r.Lk, r.qp, r.h4, r.c);
        step<true, MASK>(st, sb, sa, kl + kSB * D, vl + kSB * D, kBN * t + kSB, r.Lk, r.qp, r.h4, r.c);
    }

    // the final tile (t = n_tiles - 1): block 2t+1, if it exists, is the
    // last one, and no tile follows to be loaded
    template <int P, bool MASK>
    __device__ __forceinline__ static void tile_final(State &st, floatx16 &sa, floatx16 &sb, const Ring &r, int t)
    {
        tile_wait();
        if (CAUSAL && MASK && kBN * t > r.wlast) return;
        const _Float16 *kl = r.klds[P ^ 1], *vl = r.vlds[P];
        if (2 * t + 1 < r.n_blocks) {
            step<true, MASK>(st, sa, sb, kl, vl, kBN * t, r.Lk, r.qp, r.h4, r.c);
            step<false, MASK>(st, sb, sa, nullptr, vl + kSB * D, kBN * t + kSB, r.Lk, r.qp, r.h4, r.c);
        } else {
            step<false, MASK>(st, sa, sb, nullptr, vl, kBN * t, r.Lk, r.qp, r.h4, r.c);
        }
    }

    // tiles t .. end-1, each with a successor block; t is advanced to end.
    // The loop body is two straight-line tiles (buffer parity 0, then 1).
    template <bool MASK>
    __device__ __forceinline__ static void tiles(State &st, floatx16 &sa, floatx16 &sb, const Ring &r, int &t,
                                                 int end)
    {
        if ((t & 1) && t < end) {
            tile<1, MASK>(st, sa, sb, r, t);
            ++t;
        }
        for (; t + 1 < end; t += 2) {
            tile<0, MASK>(st, sa, sb, r, t);
            tile<1, MASK>(st, sa, sb, r, t + 1);
        }
        if (t < end) {
            tile<0, MASK>(st, sa, sb, r, t);
            ++t;
        }
    }

    template <bool MASK>
    __device__ __forceinline__ static void final_tile(State &st, floatx16 &sa, floatx16 &sb, const Ring &r, int t)
    {
        if (t & 1) tile_final<1, MASK>(st, sa, sb, r, t);
        else tile_final<0, MASK>(st, sa, sb, r, t);
    }

    // One work item: q block qb of query head h (K/V head hk) of batch b.
    __device__ __forceinline__ static void item(const Args &a, int b, int hk, int h, int qb,
                                                _Float16 (*klds)[G::kTile], _Float16 (*vlds)[G::kTile])
    {
        // In the persistent loop the thread id passes through an empty asm
        // statement once per work item, so everything derived from it is
        // computed inside the loop of `run` rather than hoisted out of it and
        // kept live (and spilled) across the whole loop.
        int tid = threadIdx.x;
        if constexpr (kPersistent) __asm__ volatile("" : "+v"(tid));
        const int lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int col = lane & 31, half = lane >> 5;
        const int Lq = a.Lq, Lk = a.Lk;
        const int q0 = qb * kBM;

        const int64_t q_row = (int64_t)a.H * D, kv_row = (int64_t)a.Hkv * D;
        const _Float16 *qbase = a.q + (int64_t)b * Lq * q_row + (int64_t)h * D;
        const _Float16 *kbase = a.k + (int64_t)b * Lk * kv_row + (int64_t)hk * D;
        const _Float16 *vbase = a.v + (int64_t)b * Lk * kv_row + (int64_t)hk * D;

        // keys the work item can see: all of them, or (causal) up to the
        // position of its last query row
        int kv_end = Lk;
        if (CAUSAL) {
            const int last = (q0 + kBM < Lq ? q0 + kBM : Lq) - 1 + a.past_len;
            kv_end = last < Lk - 1 ? last + 1 : Lk;
        }
        const int n_blocks = kv_end > 0 ? (kv_end + kSB - 1) / kSB : 0;
        const int n_tiles = kv_end > 0 ? (kv_end + kBN - 1) / kBN : 0;

        State st;
        const int wq0 = q0 + 32 * wave;
        const int qi = wq0 + col;
        // key position of this lane's query; rows past the end (never
        // written) take the last row's
        const int qp = (qi < Lq ? qi : Lq - 1) + a.past_len;
        M::init(st);

        // a work item that sees no key (every row: O = 0, LSE = -inf) skips
        // the pipeline; n_blocks is the same for the whole workgroup
        if (n_blocks > 0) {
            // K tile -1 (keys 0..31 in its upper half) and V tile 0 in flight
            // while Q is fetched
            LoadOffsets<D, W> lo;
            init_load_offsets<D, W>(lo, kv_row, tid);
            const char *k0tile = (const char *)(kbase + kSB * kv_row);
            const char *v0tile = (const char *)vbase;
            const uint32_t tile_stride = (uint32_t)(2 * kBN * kv_row);  // < 2^31 (the host checks Hkv*D)
            issue_loads<D, W, false, true>(lo, k0tile - tile_stride, kv_row, -kSB, Lk, klds[0], wave, tid);
            issue_loads<D, W, true, true>(lo, v0tile, kv_row, 0, Lk, vlds[0], wave, tid);
#pragma unroll
            for (int s = 0; s < kSteps; ++s) {
                half8 val = {};
                if (qi < Lq) val = *(const half8 *)(qbase + (int64_t)qi * q_row + 16 * s + 8 * half);
                st.qf[s] = val;
            }
            // K row = col (+ 32 for the upper half of a tile)
            M::init_lds_bases(st, lane);
            const float c = a.scale_log2;

            // prologue: scores and exact reference maximum of block 0; K tile 0 in flight
            const int wlast = __builtin_amdgcn_readfirstlane(wq0 + 31 + a.past_len);
            const Ring r{&lo, k0tile, v0tile, tile_stride, kv_row, n_tiles, n_blocks, Lk, qp, 4 * half, tid, wave, c,
                         klds, vlds, wlast};
            floatx16 sa, sb;
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (n_blocks > 1) issue_loads<D, W, false, true>(lo, k0tile, kv_row, kSB, Lk, klds[1], wave, tid);
            s_product(sa, st, klds[0] + kSB * D);
            mask(sa, 0, Lk, qp, 4 * half);
            rescale(st, block_max(sa), c);

            // Tiles t < n_main have a successor for both blocks; tile
            // n_tiles - 1 holds the last block.  The first t_clean tiles need
            // no mask on any wavefront: every key is < Lk and (causal) at or
            // before the position of the work item's first query row.
            const int n_main = (n_blocks - 1) / 2;
            int n_clean = Lk / kSB;
            if (CAUSAL) {
                const int first = q0 + a.past_len;  // position of the first query row
                const int nc = first < 0 ? 0 : (first + 1) / kSB;
                n_clean = nc < n_clean ? nc : n_clean;
            }
            const int t_clean = n_clean / 2 < n_main ? n_clean / 2 : n_main;
            int t = 0;
            tiles<false>(st, sa, sb, r, t, t_clean);
            tiles<true>(st, sa, sb, r, t, n_main);
            // the last tile needs no mask when its blocks are all clean
            if (n_blocks > n_clean) final_tile<true>(st, sa, sb, r, t);
            else final_tile<false>(st, sa, sb, r, t);
        }

        // ---- finalise: O = acc / l (guarded as on the page), LSE = scale*m + ln l
        // (a row that saw no key: acc = 0, l = 0, m = -inf -> O = 0, LSE = -inf)
        const float lt = pair_sum(st.l);
        const float inv = 1.0f / (lt > 1e-6f ? lt : 1.0f);
        // Register 4rb+J of d block i holds d = 32i + 8rb + 4*half + J.  For
        // each pair rb = 2e, 2e+1 the two lane halves exchange one packed
        // pair (v_permlane32_swap: the upper lanes of the first operand trade
        // with the lower lanes of the second), after which lane half 0 holds
        // d = 32i+16e+0..7 and half 1 holds d = 32i+16e+8..15: every lane
        // stores 16 contiguous bytes of its row, and a row's 32 bytes per
        // store instruction come from two adjacent lanes.  Lanes l and l^32
        // share a query row, so the exchange runs with every lane active.
        uint32_t ow[kDBlocks][2][4];
#pragma unroll
        for (int i = 0; i < kDBlocks; ++i)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                uint32_t w[2][2];
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int rb = 2 * e + j;
                    const float2v lo2 = {st.oacc[i][4 * rb + 0] * inv, st.oacc[i][4 * rb + 1] * inv};
                    const float2v hi2 = {st.oacc[i][4 * rb + 2] * inv, st.oacc[i][4 * rb + 3] * inv};
                    w[j][0] = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo2, half2v));
                    w[j][1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(hi2, half2v));
                }
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    const auto r = __builtin_amdgcn_permlane32_swap(w[0][x], w[1][x], false, false);
                    ow[i][e][x] = r[0];      // half 0: d +0..3, half 1: d +8..11
                    ow[i][e][2 + x] = r[1];  // half 0: d +4..7, half 1: d +12..15
                }
            }
        if (qi < Lq) {
            _Float16 *orow = a.o + (int64_t)b * Lq * q_row + (int64_t)qi * q_row + (int64_t)h * D;
#pragma unroll
            for (int i = 0; i < kDBlocks; ++i)
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const uint4v v4 = {ow[i][e][0], ow[i][e][1], ow[i][e][2], ow[i][e][3]};
                    *(uint4v *)(orow + 32 * i + 16 * e + 8 * half) = v4;
                }
            if (a.lse && half == 0)
                a.lse[((int64_t)b * a.H + h) * Lq + qi] = st.m * a.scale + __logf(lt);
        }
    }

    // Row group r = (b * Hkv + hk) * groups + g -> batch, K/V head, query head.
    __device__ __forceinline__ static void decode(const Args &a, int r, int &b, int &hk, int &h)
    {
        const int g = r % a.groups;
        r /= a.groups;
        hk = r % a.Hkv;
        b = r / a.Hkv;
        h = hk * a.groups + g;
    }

    // Work decomposition.
    //  * Full pass: one workgroup per work item, xcd_item(blockIdx.x).
    //  * Causal (the loop of the pages' kernel over q blocks): persistent.  The
    //    grid is the resident workgroups, a multiple of 8, and the work items
    //    are single q blocks, whose cost falls with the block index.  The row
    //    groups are cut into 8 contiguous ranges, one per XCD (workgroups
    //    reach the XCDs round robin), so that the query heads sharing a K/V
    //    head stay in one L2.  An XCD walks its range in phases of C row
    //    groups; a phase's items are ordered heaviest first (q block nQ-1 of
    //    each of its row groups, then nQ-2, ...) and dealt to the XCD's gx
    //    workgroups in rounds whose direction alternates, so the workgroup
    //    that takes the heaviest item of one round takes the lightest of the
    //    next.  C is the fewest row groups whose items fill an even number of
    //    rounds (2 gx / gcd(nQ, 2 gx), from the host), which balances every
    //    phase exactly while only C row groups' K/V are in use at a time;
    //    where C does not divide the range, one phase covers it all (balanced
    //    to within one item).  With fewer than 8 row groups the whole grid
    //    deals all items the same way.  A barrier separates consecutive
    //    items, whose first loads reuse the LDS tiles.
    __device__ static void run(const Args &a)
    {
        __shared__ __attribute__((aligned(16))) _Float16 klds[2][G::kTile];
        __shared__ __attribute__((aligned(16))) _Float16 vlds[2][G::kTile];
        const int nq = a.n_qblocks;
        if constexpr (!kPersistent) {
            const int it = xcd_item(blockIdx.x, a.n_items);
            int b, hk, h;
            decode(a, it / nq, b, hk, h);
            item(a, b, hk, h, it % nq, klds, vlds);
        } else {
            int gx = (int)gridDim.x, s = (int)blockIdx.x, rg0 = 0, nrg = a.n_rows;
            if (a.n_rows >= kXcds) {
                const int x = (int)blockIdx.x % kXcds, per = a.n_rows / kXcds, extra = a.n_rows % kXcds;
                rg0 = x * per + (x < extra ? x : extra);
                nrg = per + (x < extra ? 1 : 0);
                gx /= kXcds;
                s /= kXcds;
            }
            const int C = nrg % a.phase_rows == 0 ? a.phase_rows : nrg;
            // With several phases, the slots that take one row group's items
            // in a round are made consecutive (slot s deals as s'), which
            // spreads a row group over the XCD's compute units (measured:
            // HBM reads of the causal B=8 H=32 L=4096 pass -31 %, 2 % faster;
            // a single phase keeps the plain order, 5 % faster at D = 64)
            if (C < nrg && gx % C == 0) {
                const int m = gx / C;
                s = (s % m) * C + s / m;
            }
            bool started = false;
            for (int p0 = 0; p0 < nrg; p0 += C) {
                const int n = C * nq;  // this phase's items
                for (int r = 0;; ++r) {
                    const int idx = r * gx + ((r & 1) ? gx - 1 - s : s);  // < items + grid < 2^31
                    if (idx >= n) break;  // every later round starts past n as well
                    int b, hk, h;
                    decode(a, rg0 + p0 + idx % C, b, hk, h);
                    if (started) __syncthreads();  // every wavefront is done with the LDS tiles
                    started = true;
                    item(a, b, hk, h, nq - 1 - idx / C, klds, vlds);
                }
            }
        }
    }
};

// Wavefronts per SIMD: 2 at D = 128 (about 248 VGPRs each); 3 at D = 64,
// whose 164 VGPRs and 32 KiB of LDS per four-wavefront workgroup let three
// workgroups share a CU (measured 12-14 % faster than 2 on the B=8, H=32,
// L=1024 workloads; 4 per SIMD would need 128 VGPRs and spills).
template <int D, bool CAUSAL, int W>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * W, 64 * W),
                          amdgpu_waves_per_eu(D == 64 ? 3 : 2, D == 64 ? 3 : 2))) void
fa_fwd_kernel(const Args a)
{
    Kernel<D, CAUSAL, W>::run(a);
}

// Workgroups of `kernel` (with `threads` threads) resident on the whole
// current device at once: compute units x workgroups per compute unit (from
// the kernel's registers and LDS).  Queried once per device and kernel; 0 if
// the runtime cannot say.
int resident_workgroups(const void *kernel, int threads)
{
    constexpr int kMaxDevices = 64, kMaxKernels = 8;
    static std::atomic<int> cache[kMaxDevices][kMaxKernels];
    static std::atomic<const void *> keys[kMaxKernels];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    int slot = -1;
    for (int i = 0; i < kMaxKernels && slot < 0; ++i) {
        const void *cur = keys[i].load();
        if (cur == kernel) slot = i;
        else if (cur == nullptr) {
            const void *expected = nullptr;
            if (keys[i].compare_exchange_strong(expected, kernel) || expected == kernel) slot = i;
        }
    }
    if (slot >= 0 && dev < kMaxDevices) {
        const int v = cache[dev][slot].load();
        if (v > 0) return v;
    }
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess) return 0;
    const int v = cus > 0 && per_cu > 0 ? cus * per_cu : 0;
    if (slot >= 0 && dev < kMaxDevices && v > 0) cache[dev][slot].store(v);
    return v;
}

template <int D, bool CAUSAL, int W>
int launch_w(Args args, hipStream_t stream)
{
    using K = Kernel<D, CAUSAL, W>;
    args.n_qblocks = (args.Lq + K::kBM - 1) / K::kBM;
    const int64_t items = (int64_t)args.n_items * args.n_qblocks;  // n_items holds B*H here
    // the persistent schedule's item indices stay below items + grid; no
    // problem that fits in memory comes near this bound
    if (items > (1 << 30)) return FA_ERR_SHAPE;
    const int rows = args.n_items;
    args.n_items = (int)items;
    int grid = args.n_items;
    args.n_rows = rows;
    args.phase_rows = 1;
    if (K::kPersistent) {
        const int slots = resident_workgroups((const void *)fa_fwd_kernel<D, CAUSAL, W>, K::kThreads);
        if (slots <= 0) return FA_ERR_DEVICE;
        // a multiple of 8, so that blockIdx.x % 8 names the XCD for every slot
        const int64_t want = items < slots ? items : slots;
        grid = (int)((want + kXcds - 1) / kXcds * kXcds);
        const int gx2 = 2 * (rows >= kXcds ? grid / kXcds : grid);
        args.phase_rows = gx2 / std::gcd(args.n_qblocks, gx2);
    }
    if (grid == 0) return FA_OK;
    hipLaunchKernelGGL((fa_fwd_kernel<D, CAUSAL, W>), dim3(grid), dim3(K::kThreads), 0, stream, args);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// Wavefronts per workgroup, measured per workload (same-process A/B): 8 for
// the full pass at D = 128 (each K/V tile serves 256 queries); 4 at D = 64
// and under the causal mask, where a 256-row block leaves half its
// wavefronts computing masked blocks along the diagonal -- except from 4096
// keys on, where the diagonal is a small share of a work item and halving
// the K/V tile traffic per flop wins (measured: W = 4 is 4-25 % faster at
// 512-2048 keys, W = 8 about 1 % at 4096 and 3 % for 1024 queries after
// 3072 cached keys).
template <int D, bool CAUSAL>
int launch(Args args, hipStream_t stream)
{
    if constexpr (D == 128 && CAUSAL) {
        if (args.Lk >= 4096) return launch_w<D, CAUSAL, 8>(args, stream);
        return launch_w<D, CAUSAL, 4>(args, stream);
    } else {
        return launch_w<D, CAUSAL, (D == 64 ? 4 : 8)>(args, stream);
    }
}

}  // namespace

int launch_forward(const Problem &p, hipStream_t stream)
{
    // per-lane tile offsets are 32-bit: a tile of kBN K/V rows must span < 2 GiB
    if ((int64_t)p.Hkv * p.D * 2 * kBN > 0x7fffffff) return FA_ERR_SHAPE;
    const int64_t bh = (int64_t)p.B * p.H;
    if (bh > 0x7fffffff) return FA_ERR_SHAPE;
    Args a;
    a.q = (const _Float16 *)p.q;
    a.k = (const _Float16 *)p.k;
    a.v = (const _Float16 *)p.v;
    a.o = (_Float16 *)p.o;
    a.lse = p.lse;
    a.Lq = p.Lq;
    a.Lk = p.Lk;
    a.past_len = p.past_len;
    a.H = p.H;
    a.Hkv = p.Hkv;
    a.groups = p.H / p.Hkv;
    a.n_qblocks = 0;
    a.n_items = (int)bh;
    a.scale = p.scale;
    a.scale_log2 = p.scale * 1.4426950408889634f;
    if (p.D == 64) return p.causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
    return p.causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
}

}  // namespace fa