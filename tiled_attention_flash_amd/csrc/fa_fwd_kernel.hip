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
//   the full (non-causal) pass -- each K/V tile brought into LDS then serves
//   256 queries -- and W = 4 under the causal mask, where the smaller block
//   keeps the wavefronts of a workgroup evenly loaded along the diagonal.
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
//   one is computed.  The source address of each lane is chosen so that rows
//   land with a 16-byte-chunk XOR swizzle that makes the K reads
//   (ds_read_b128, 16 rows per LDS cycle) and the V transpose reads (4 rows x
//   64 bytes per half-wavefront) free of bank conflicts.  Rows past the end
//   of the sequence load row L-1 instead (finite data that the mask hides).
// * Online softmax with a lazy rescale: the reference maximum of a row is
//   raised (and O, l rescaled) only when some row of the wavefront sees its
//   maximum grow by more than 2^8 in the exp2 domain; otherwise the stale
//   maximum keeps every probability <= 256 (well inside fp16's range) and the
//   final O / l and LSE are unchanged.
// * Causal: tiles past the block's last query are never visited; the mask
//   code runs only on tiles that straddle a wavefront's diagonal (or hold the
//   ragged end of the sequence).
// * Grid: one workgroup per (b, kv head, group member, q block) work item;
//   workgroup ids are remapped so that each of the 8 XCDs (which receive
//   workgroups round-robin) walks a contiguous range of work items, keeping
//   one head's K/V in that XCD's L2.  Causal q blocks run heaviest first.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_internal.h"

namespace fa {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float float2v __attribute__((ext_vector_type(2)));

#define LDS_AS __attribute__((address_space(3)))

constexpr int kBN = 64;               // keys per K/V tile
constexpr int kKB = kBN / 32;         // 32-key blocks of S^T per tile
constexpr int kCS = kBN / 16;         // 16-key k-steps of the P.V product per tile
constexpr int kXcds = 8;
constexpr float kRescaleLog2 = 8.0f;  // lazy-rescale threshold (exp2 domain)

struct Args {
    const _Float16 *q, *k, *v;
    _Float16 *o;
    float *lse;
    int L, H, Hkv, groups, n_qblocks, n_items;
    float scale;       // multiplier of Q.K
    float scale_log2;  // scale * log2(e): exp(scale*x) == exp2(scale_log2*x)
};

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// v_permlane32_swap exchanges the upper half of one register with the lower
// half of another; given the same value twice, each lane ends up holding its
// own value in one result and lane l^32's value in the other, so a symmetric
// combination of the two is the cross-half max / sum.
__device__ __forceinline__ float pair_max(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

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

// Physical 16-byte chunk of logical chunk `c` of K row `row`: 16 consecutive
// rows read at one logical chunk hit 16 distinct 16-byte bank groups.
template <int D>
__device__ __forceinline__ int k_chunk(int row, int c)
{
    return D == 128 ? (c ^ (row & 15)) : (c ^ ((row >> 1) & 7));
}

// Physical chunk for V rows: the 4 rows x 64 bytes a half-wavefront
// transpose-reads at once land in distinct bank groups.
template <int D>
__device__ __forceinline__ int v_chunk(int row, int c)
{
    return D == 128 ? (c ^ ((row & 3) << 2)) : (c ^ (((row >> 1) & 1) << 2));
}

// Tile row that this lane's n-th direct load fills.
template <int D, int W>
__device__ __forceinline__ int load_row(int n)
{
    using G = Geo<D, W>;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
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
__device__ __forceinline__ void init_load_offsets(LoadOffsets<D, W> &lo, int64_t kv_row)
{
    using G = Geo<D, W>;
    const int pc = (threadIdx.x & 63) % G::kChunks;
#pragma unroll
    for (int n = 0; n < G::kLoadsPerWave; ++n) {
        const int row = load_row<D, W>(n);
        lo.k[n] = (uint32_t)(2 * (row * kv_row + 8 * k_chunk<D>(row, pc)));
        lo.v[n] = (uint32_t)(2 * (row * kv_row + 8 * v_chunk<D>(row, pc)));
    }
}

// One 16-byte-per-lane direct HBM -> LDS load: lane i's 16 bytes from
// base + off land at lds + 16*i.  Written as inline assembly so that the
// compiler does not see the LDS tile buffers as written by an in-flight load
// and stall every later LDS read until all loads complete (it cannot tell
// the two buffers apart); the kernel itself waits for a tile's loads before
// the barrier that hands the tile to the workgroup.
__device__ __forceinline__ void dma16(const char *base, uint32_t off, _Float16 *lds)
{
    const uint32_t m0 = (uint32_t)(uintptr_t)(LDS_AS void *)lds;
    __asm__ volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                     :
                     : "v"(off), "s"(base), "{m0}"(m0)
                     : "memory");
}

// Issue this wave's share of the direct loads of the K and V tiles that start
// at key k0.  A tile reaching past L loads row L-1 in place of the missing
// rows (finite data that the mask hides).
template <int D, int W>
__device__ __forceinline__ void issue_tile_loads(const LoadOffsets<D, W> &lo,
                                                 const _Float16 *kbase, const _Float16 *vbase,
                                                 int64_t kv_row, int k0, int L, _Float16 *klds,
                                                 _Float16 *vlds)
{
    using G = Geo<D, W>;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const char *kt = (const char *)(kbase + (int64_t)k0 * kv_row);
    const char *vt = (const char *)(vbase + (int64_t)k0 * kv_row);
    const bool full = k0 + kBN <= L;
#pragma unroll
    for (int n = 0; n < G::kLoadsPerWave; ++n) {
        const int blk = G::kLoadsPerWave * wave + n;
        uint32_t ko = lo.k[n], vo = lo.v[n];
        if (!full) {
            const int over = k0 + load_row<D, W>(n) - (L - 1);  // rows past the end re-read row L-1
            if (over > 0) {
                ko -= (uint32_t)(2 * over * kv_row);
                vo -= (uint32_t)(2 * over * kv_row);
            }
        }
        dma16(kt, ko, klds + 512 * blk);
        dma16(vt, vo, vlds + 512 * blk);
    }
}

__device__ __forceinline__ half8 lds_read16(const _Float16 *p) { return *(const half8 *)p; }

__device__ __forceinline__ half4 lds_read_tr(const _Float16 *p)
{
    short4v v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS short4v *)(p));
    return __builtin_bit_cast(half4, v);
}

// Work item -> position in the (b, kv head, group member, q block) order.
__device__ __forceinline__ int xcd_item(int block, int n)
{
    int x = block % kXcds, slot = block / kXcds;
    int per = n / kXcds, extra = n % kXcds;
    return x * per + (x < extra ? x : extra) + slot;
}

template <int D, bool CAUSAL, int W>
struct Kernel {
    using G = Geo<D, W>;
    static constexpr int kThreads = 64 * W;
    static constexpr int kBM = 32 * W;       // query rows per work item
    static constexpr int kSteps = D / 16;    // k-steps of S^T = K.Q^T
    static constexpr int kDBlocks = D / 32;  // 32-row blocks of O^T

    // per-lane state of one wavefront
    struct State {
        half8 qf[kSteps];
        floatx16 oacc[kDBlocks];
        float m;     // reference row maximum (raw score units)
        float l;     // running row sum, this lane's keys
        int k_base;  // LDS half offset of this lane's K read at k-step 0
        int v_base;  // LDS half offset of this lane's V transpose read at d block 0
    };

    // The swizzles are XORs on the 16-byte chunk index, and the chunk index
    // of k-step s (d block i) differs from that of step 0 (block 0) only in
    // bits the XOR touches, so each read address is one XOR from the base.
    __device__ __forceinline__ static int k_offset(const State &st, int s) { return st.k_base ^ (16 * s); }
    __device__ __forceinline__ static int v_offset(const State &st, int i) { return st.v_base ^ (32 * i); }

    // S^T = K . Q^T for the 64 keys of the tile, as two 32-key blocks;
    // every K fragment of the tile is requested before the first MFMA so LDS
    // latency is paid once per tile, not once per k-step
    static constexpr int kAhead = kSteps;

    __device__ __forceinline__ static void s_product(floatx16 (&sacc)[kKB], const State &st,
                                                     const _Float16 *kl)
    {
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb) sacc[kb] = floatx16{};
        half8 ka[kSteps][kKB];
#pragma unroll
        for (int s = 0; s < kAhead; ++s)
#pragma unroll
            for (int kb = 0; kb < kKB; ++kb) ka[s][kb] = lds_read16(kl + k_offset(st, s) + 32 * kb * D);
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
            if (s + kAhead < kSteps)
#pragma unroll
                for (int kb = 0; kb < kKB; ++kb)
                    ka[s + kAhead][kb] = lds_read16(kl + k_offset(st, s + kAhead) + 32 * kb * D);
#pragma unroll
            for (int kb = 0; kb < kKB; ++kb)
                sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[s][kb], st.qf[s], sacc[kb], 0, 0, 0);
        }
    }

    // mask, row maximum, lazy rescale, and P = exp2(S*c - m*c) as fp16 B
    // operands of the P.V product (one per 16-key k-step), with the row sum
    __device__ __forceinline__ static void softmax(State &st, floatx16 (&sacc)[kKB], half8 (&pf)[kCS],
                                                   int k0, int L, int wq0, int qi, float c)
    {
        const int half = (threadIdx.x & 63) >> 5;

        // mask: keys past the sequence end, and keys after the query (causal).
        // Register r of block kb holds key k0 + 4*half + 32kb + 8(r/4) + r%4,
        // so one per-lane bound decides every element.
        if ((k0 + kBN > L) || (CAUSAL && k0 + kBN - 1 > wq0)) {
            int bound = L - k0 - 4 * half;  // hide offsets >= bound
            if (CAUSAL) {
                const int cb = qi - k0 - 4 * half + 1;
                bound = cb < bound ? cb : bound;
            }
#pragma unroll
            for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (32 * kb + 8 * (r >> 2) + (r & 3) >= bound) sacc[kb][r] = -__builtin_huge_valf();
        }

        // row maximum of the tile, both lane halves: four independent chains
        // (short dependency chains), then one cross-half exchange
        float mq[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) mq[a] = sacc[0][a];
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
            for (int r = (kb == 0 ? 4 : 0); r < 16; ++r) mq[r & 3] = fmaxf(mq[r & 3], sacc[kb][r]);
        float mx = fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3]));
        mx = pair_max(mx);

        // lazy rescale: raise the reference maximum only when some row's
        // maximum outgrew it by more than 2^kRescaleLog2
        const bool grow = (mx - st.m) * c > kRescaleLog2;
        if (__builtin_amdgcn_ballot_w64(grow)) {
            const float m_new = fmaxf(st.m, mx);
            const float sf = exp2_fast((st.m - m_new) * c);
            st.l *= sf;
#pragma unroll
            for (int i = 0; i < kDBlocks; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) st.oacc[i][r] *= sf;
            st.m = m_new;
        }
        const float mc = st.m * c;

        // P = exp2(S*c - m*c) as fp16 B operands (round-to-nearest-even), one
        // per 16-key k-step.  The row sum adds up exactly those fp16 values
        // (the weights the P.V product applies), two per v_dot2_f32_f16 into
        // fp32, in four partial sums (partial sum a = 2(cs&1) + e/4 is first
        // written at cs < 2, e in {0,4})
        float rs[4];
#pragma unroll
        for (int cs = 0; cs < kCS; ++cs)
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const int kb = cs >> 1, r = 8 * (cs & 1) + e;
                const float p0 = exp2_fast(__builtin_fmaf(sacc[kb][r], c, -mc));
                const float p1 = exp2_fast(__builtin_fmaf(sacc[kb][r + 1], c, -mc));
                const int a = (cs & 1) * 2 + (e >> 2);
                const float2v f2 = {p0, p1};
                const half2v h2 = __builtin_convertvector(f2, half2v);
                const half2v ones = {(_Float16)1.0f, (_Float16)1.0f};
                if (cs < 2 && (e & 3) == 0) rs[a] = __builtin_amdgcn_fdot2(h2, ones, 0.0f, false);
                else rs[a] = __builtin_amdgcn_fdot2(h2, ones, rs[a], false);
                pf[cs][e] = h2[0];
                pf[cs][e + 1] = h2[1];
            }
        st.l += (rs[0] + rs[1]) + (rs[2] + rs[3]);
    }

    // O^T += V^T . P^T ; the A operand of k-step cs is two transpose reads:
    // keys 16cs + 4h + 0..3 and 16cs + 8 + 4h + 0..3 for lane half h.  The
    // reads of d block i+1 are in flight during the MFMAs of block i.
    __device__ __forceinline__ static void pv_product(State &st, const half8 (&pf)[kCS],
                                                      const _Float16 *vl)
    {
        // MFMA n = (d block i, k-step cs) = (n / kCS, n % kCS); its operand is
        // read kVAhead MFMAs earlier
        constexpr int kN = kDBlocks * kCS;
        constexpr int kVAhead = 4;
        half8 va[kN];
        auto vload = [&](int n) {
            const _Float16 *vi = vl + v_offset(st, n / kCS);
            const int cs = n % kCS;
            const half4 lo = lds_read_tr(vi + 16 * cs * D);
            const half4 hi = lds_read_tr(vi + (16 * cs + 8) * D);
            va[n] = half8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        };
#pragma unroll
        for (int n = 0; n < kVAhead; ++n) vload(n);
#pragma unroll
        for (int n = 0; n < kN; ++n) {
            if (n + kVAhead < kN) vload(n + kVAhead);
            st.oacc[n / kCS] =
                __builtin_amdgcn_mfma_f32_32x32x16_f16(va[n], pf[n % kCS], st.oacc[n / kCS], 0, 0, 0);
        }
    }

    // one whole K/V tile for one wavefront
    __device__ __forceinline__ static void tile(State &st, const _Float16 *kl, const _Float16 *vl,
                                                int k0, int L, int wq0, int qi, float c)
    {
        floatx16 sacc[kKB];
        half8 pf[kCS];
        s_product(sacc, st, kl);
        softmax(st, sacc, pf, k0, L, wq0, qi, c);
        pv_product(st, pf, vl);
    }

    __device__ static void run(const Args &a)
    {
        __shared__ __attribute__((aligned(16))) _Float16 klds[2][G::kTile];
        __shared__ __attribute__((aligned(16))) _Float16 vlds[2][G::kTile];

        const int tid = threadIdx.x;
        const int lane = tid & 63, wave = tid >> 6;
        const int col = lane & 31, half = lane >> 5;

        // ---- work item
        const int item = xcd_item(blockIdx.x, a.n_items);
        int rest = item / a.n_qblocks;
        int qb = item % a.n_qblocks;
        if (CAUSAL) qb = a.n_qblocks - 1 - qb;  // heaviest blocks first
        const int g = rest % a.groups;
        rest /= a.groups;
        const int hk = rest % a.Hkv;
        const int b = rest / a.Hkv;
        const int h = hk * a.groups + g;
        const int L = a.L;
        const int q0 = qb * kBM;

        const int64_t q_row = (int64_t)a.H * D, kv_row = (int64_t)a.Hkv * D;
        const _Float16 *qbase = a.q + (int64_t)b * L * q_row + (int64_t)h * D;
        const _Float16 *kbase = a.k + (int64_t)b * L * kv_row + (int64_t)hk * D;
        const _Float16 *vbase = a.v + (int64_t)b * L * kv_row + (int64_t)hk * D;

        const int kv_end = CAUSAL ? (q0 + kBM < L ? q0 + kBM : L) : L;
        const int n_tiles = (kv_end + kBN - 1) / kBN;

        // first tile in flight while Q is fetched
        LoadOffsets<D, W> lo;
        init_load_offsets<D, W>(lo, kv_row);
        issue_tile_loads<D, W>(lo, kbase, vbase, kv_row, 0, L, klds[0], vlds[0]);

        State st;
        const int wq0 = q0 + 32 * wave;
        const int qi = wq0 + col;
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
            half8 val = {};
            if (qi < L) val = *(const half8 *)(qbase + (int64_t)qi * q_row + 16 * s + 8 * half);
            st.qf[s] = val;
        }
#pragma unroll
        for (int i = 0; i < kDBlocks; ++i) st.oacc[i] = floatx16{};
        st.m = -__builtin_huge_valf();
        st.l = 0.0f;
        // K: row = 32*kb + col, logical chunk 2s + half
        st.k_base = col * D + 8 * k_chunk<D>(col, half);
        // V transpose read: 16-lane group gg = lane/16 (d half gg%2, key half
        // gg/2), j = lane%16 -> row 4*(gg/2) + j/4 (+ 16*cs [+ 8]),
        // d = 32*i + 16*(gg%2) + 4*(j%4)
        {
            const int gg = lane >> 4, j = lane & 15;
            const int row = 4 * (gg >> 1) + (j >> 2);
            const int d = 16 * (gg & 1) + 4 * (j & 3);
            st.v_base = row * D + 8 * v_chunk<D>(row, d >> 3) + (d & 7);
        }

        const float c = a.scale_log2;
        for (int t = 0; t < n_tiles; t += 2) {
            step<0>(st, lo, kbase, vbase, kv_row, t, n_tiles, L, wq0, qi, c, klds, vlds);
            if (t + 1 < n_tiles)
                step<1>(st, lo, kbase, vbase, kv_row, t + 1, n_tiles, L, wq0, qi, c, klds, vlds);
        }

        // ---- finalise: O = acc / l (guarded as on the page), LSE = scale*m + ln l
        const float lt = pair_sum(st.l);
        const float inv = 1.0f / (lt > 1e-6f ? lt : 1.0f);
        if (qi < L) {
            _Float16 *orow = a.o + (int64_t)b * L * q_row + (int64_t)qi * q_row + (int64_t)h * D;
#pragma unroll
            for (int i = 0; i < kDBlocks; ++i)
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    const float2v lo2 = {st.oacc[i][4 * rb + 0] * inv, st.oacc[i][4 * rb + 1] * inv};
                    const float2v hi2 = {st.oacc[i][4 * rb + 2] * inv, st.oacc[i][4 * rb + 3] * inv};
                    const half2v hl = __builtin_convertvector(lo2, half2v);
                    const half2v hh = __builtin_convertvector(hi2, half2v);
                    const half4 out = {hl[0], hl[1], hh[0], hh[1]};
                    *(half4 *)(orow + 32 * i + 8 * rb + 4 * half) = out;
                }
            if (a.lse && half == 0)
                a.lse[((int64_t)b * a.H + h) * L + qi] = st.m * a.scale + __logf(lt);
        }
    }

    // One K/V tile: wait for its loads, barrier, start the next tile's loads
    // into the other buffer, compute.  BUF is the buffer tile t lives in.
    template <int BUF>
    __device__ __forceinline__ static void step(State &st, const LoadOffsets<D, W> &lo,
                                                const _Float16 *kbase, const _Float16 *vbase,
                                                int64_t kv_row, int t, int n_tiles, int L,
                                                int wq0, int qi, float c,
                                                _Float16 (*klds)[G::kTile],
                                                _Float16 (*vlds)[G::kTile])
    {
        __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of tile t have landed
        __syncthreads();                // ... and every wave's; tile t-1 fully consumed
        if (t + 1 < n_tiles)
            issue_tile_loads<D, W>(lo, kbase, vbase, kv_row, (t + 1) * kBN, L, klds[BUF ^ 1],
                                   vlds[BUF ^ 1]);
        const int k0 = t * kBN;
        // a wavefront whose 32 queries all precede this tile has nothing to do
        if (!CAUSAL || k0 <= wq0 + 31) tile(st, klds[BUF], vlds[BUF], k0, L, wq0, qi, c);
    }
};

template <int D, bool CAUSAL, int W>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * W, 64 * W),
                          amdgpu_waves_per_eu(2, 2))) void
fa_fwd_kernel(const Args a)
{
    Kernel<D, CAUSAL, W>::run(a);
}

template <int D, bool CAUSAL>
int launch(Args args, hipStream_t stream)
{
    constexpr int W = CAUSAL ? 4 : 8;
    using K = Kernel<D, CAUSAL, W>;
    args.n_qblocks = (args.L + K::kBM - 1) / K::kBM;
    const int64_t items = (int64_t)args.n_items * args.n_qblocks;  // n_items holds B*H here
    if (items > 0x7fffffff) return FA_ERR_SHAPE;
    args.n_items = (int)items;
    hipLaunchKernelGGL((fa_fwd_kernel<D, CAUSAL, W>), dim3(args.n_items), dim3(K::kThreads), 0,
                       stream, args);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
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
    a.L = p.L;
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
