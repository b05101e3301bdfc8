// fa_fwd_fp8_kernel.hip -- attention forward on FP8 (E4M3) inputs for gfx950.
//
// Method: as fa_fwd_kernel.hip (page "使用 TileLang 在 AMD GPU 上快速开发高性能
// Flash Attention", sections "Q Tile 处理与缓存初始化", "K/V Tile 遍历与核心计算"
// and "最终输出写回与Q tile 迭代"), with the 8-bit inputs that page
// "TileLang性能分析报告：H100上FlashAttention吞吐量达1.2PFlops", section
// "生产环境部署建议", names as the next step for throughput.  Q, K and V are
// OCP E4M3 codes with one descale factor per tensor; O is fp16 and the
// log-sum-exp fp32, as in the fp16 kernel.
//
// Mapping onto CDNA4
// ------------------
// * Both products run on v_mfma_f32_32x32x64_f8f6f4 (E4M3 x E4M3, fp32
//   accumulate; twice the fp16 rate), transposed as in the fp16 kernel:
//     S^T[key][query]  = K . Q^T    (A = K rows from LDS, B = Q in VGPRs)
//     O^T[d][query]   += V^T . P^T  (A = V^T from LDS,   B = P in VGPRs)
//   Lane l holds A[l%32][32(l/32) + i] and B[32(l/32) + i][l%32] for bytes
//   i = 0..31 of its 8 operand registers; the 32x32 result has the fp16
//   MFMA's layout (lane l: column l%32, rows 8I + 4(l/32) + J in register
//   4I + J).
// * The score block is 64 keys -- the 64-deep contraction of the P.V
//   product -- held as two 32x32 S^T accumulators (keys 0..31, 32..63).  The
//   32 probabilities a lane holds, converted to E4M3 in register order
//   (accumulator 0, then 1), are its B operand bytes; byte 16a + 4I + J then
//   stands for key 32a + 8I + 4h + J (h = l/32).  ds_read_b64_tr_b8 (lane j
//   of a 16-lane group receives byte j%8 of the 8-byte pieces that lanes
//   2b + j/8, b = 0..7, point at) gathers V^T in exactly that key order when
//   lanes 2b, 2b+1 of a group point at the two 8-byte halves of 16 columns of
//   key row 16t + 4h + (b&3) + 8(b>>2), read t = 0..3.
// * K/V tiles of 64 rows (one score block) travel HBM -> LDS with
//   global_load_lds_dwordx4, double-buffered, K one tile ahead of V, with one
//   workgroup barrier per tile.  One XOR swizzle of the 16-byte chunk index
//   keeps both the K reads (ds_read_b128, 16 rows at one chunk) and the V
//   transpose reads (8 rows x 2 chunks per half-wavefront) free of bank
//   conflicts.
// * Online softmax as in the fp16 kernel: block 0 sets each row's reference
//   maximum exactly; later blocks are exponentiated against it, and a block
//   whose probabilities reach the E4M3 range limit in some lane is computed
//   again after the reference is raised.  The probabilities are stored as
//   2^3 * P: the maximum's weight 8 sits well inside E4M3's normal range
//   (2^-6 .. 448), weights down to 2^-9 keep full relative precision, and a
//   lane's 32 weights sum to at most 256 < 448 while the reference is the
//   row's maximum.  The row sum adds the fp32 probabilities, so the LSE does
//   not see the E4M3 rounding.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

typedef int int8v __attribute__((ext_vector_type(8)));
typedef int int4v __attribute__((ext_vector_type(4)));
typedef int int2v __attribute__((ext_vector_type(2)));

constexpr int kBlk = 64;              // keys per score block and per LDS tile
constexpr float kOffsetLog2 = 3.0f;   // probabilities are stored as 2^3 * P
constexpr float kE4M3Max = 448.0f;    // largest finite E4M3 value
constexpr float kLn2 = 0.69314718055994531f;

struct Args8 {
    const uint8_t *q, *k, *v;
    _Float16 *o;
    float *lse;
    int Lq, Lk;
    int past_len;
    int H, Hkv, groups, n_qblocks, n_items;
    float c;          // scale * q_descale * k_descale * log2(e): exp(s) = exp2(c * raw)
    float lse_scale;  // scale * q_descale * k_descale
    float v_descale;
};

// Physical 16-byte chunk of logical chunk c of a tile row (D bytes).  The
// XOR uses row bits 1..3 (D = 128) or 2..3 (D = 64): 16 consecutive rows at
// one chunk -- a K read -- fall in 16 distinct bank groups, and so do the 8
// rows {0,1,2,3,8,9,10,11} (+4h) x 2 chunks of a half-wavefront's V
// transpose read.
template <int D>
__device__ __forceinline__ int f8_swz(int row)
{
    return D == 128 ? (((row >> 2) & 1) | (((row >> 1) & 1) << 1) | (((row >> 3) & 1) << 2))
                    : (((row >> 2) & 1) | (((row >> 3) & 1) << 1));
}

template <int D, int W>
struct Geo8 {
    static constexpr int kChunks = D / 16;             // 16-byte chunks per row
    static constexpr int kRowsPerLoad = 64 / kChunks;  // rows one wave-wide load fills (1 KiB)
    static constexpr int kLoadsPerTile = kBlk / kRowsPerLoad;
    static constexpr int kLoadsPerWave = (kLoadsPerTile + W - 1) / W;
    static constexpr int kTile = kBlk * D;  // bytes per K (or V) tile
};

// Tile row that this lane's n-th load fills (load instruction wave + W*n).
template <int D, int W>
__device__ __forceinline__ int load_row8(int wave, int n)
{
    using G = Geo8<D, W>;
    return G::kRowsPerLoad * (wave + W * n) + (threadIdx.x & 63) / G::kChunks;
}

// Issue this wave's share of the direct loads of the tile at key k0, whose
// key row 0 is at `tile`.  EDGE: the tile may reach past Lk; rows past the
// end re-read row Lk - 1 (finite data that the mask hides).  offs[n]: byte
// offset of this lane's chunk of load n relative to the tile.
template <int D, int W, bool EDGE>
__device__ __forceinline__ void issue_tile8(const uint32_t (&offs)[Geo8<D, W>::kLoadsPerWave],
                                            const char *tile, int64_t kv_row, int k0, int Lk, uint8_t *lds)
{
    using G = Geo8<D, W>;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int n = 0; n < G::kLoadsPerWave; ++n) {
        const int blk = wave + W * n;
        if (G::kLoadsPerTile % W != 0 && blk >= G::kLoadsPerTile) continue;  // wave-uniform
        uint32_t off = offs[n];
        if constexpr (EDGE) {
            const int over = k0 + load_row8<D, W>(wave, n) - (Lk - 1);
            if (over > 0) off -= (uint32_t)(over * kv_row);
        }
        dma16(tile, off, (_Float16 *)(lds + 1024 * blk));
    }
}

// The tile at key k0 = kBlk * j: its first row lies j * kBlk * kv_row bytes
// past the head's key 0 (kBlk * kv_row < 2^31, checked on the host).
template <int D, int W>
__device__ __forceinline__ void issue_tile8_at(const uint32_t (&offs)[Geo8<D, W>::kLoadsPerWave],
                                               const uint8_t *base, int64_t kv_row, int j, int Lk, uint8_t *lds)
{
    const char *tile = (const char *)base + (int64_t)j * (uint32_t)(kBlk * kv_row);
    const int k0 = kBlk * j;
    if (k0 + kBlk <= Lk) issue_tile8<D, W, false>(offs, tile, kv_row, k0, Lk, lds);
    else issue_tile8<D, W, true>(offs, tile, kv_row, k0, Lk, lds);
}

template <int D, bool CAUSAL, int W>
struct Kernel8 {
    using G = Geo8<D, W>;
    static constexpr int kS = D / 64;        // 64-deep k-steps of S^T per 32-key half
    static constexpr int kDBlocks = D / 32;  // 32-row blocks of O^T
    static constexpr int kBM = 32 * W;       // query rows per work item
    static constexpr int kThreads = 64 * W;

    struct State {
        int8v qf[kS];
        floatx16 oacc[kDBlocks];
        float m;   // reference row maximum (raw score units)
        float mc;  // m * c - 3 (0 - 3 while m = -inf)
        float l;   // row sum of 2^3 * P, this lane's keys
        int kb;    // LDS byte offset of this lane's K read (row = col, chunk 2h)
        int vb;    // LDS byte offset of this lane's V transpose read t = 0, d block 0
    };

    __device__ __forceinline__ static void init(State &st)
    {
#pragma unroll
        for (int i = 0; i < kDBlocks; ++i) st.oacc[i] = floatx16{};
        st.m = -__builtin_huge_valf();
        st.mc = -kOffsetLog2;
        st.l = 0.0f;
        const int lane = threadIdx.x & 63, col = lane & 31, h = lane >> 5;
        st.kb = col * D + 16 * ((2 * h) ^ f8_swz<D>(col));
        const int g = lane >> 4, m = lane & 15, b = m >> 1, e = m & 1;
        const int row0 = 4 * h + (b & 3) + 8 * (b >> 2);
        st.vb = row0 * D + 16 * ((g & 1) ^ f8_swz<D>(row0)) + 8 * e;
    }

    // A operand of S^T: K rows 32a + col, bytes 64s + 32h .. +31
    __device__ __forceinline__ static int8v kfrag(const State &st, const uint8_t *kl, int a, int s)
    {
        const uint8_t *p = kl + 32 * a * D;
        const int4v lo = *(const int4v *)(p + (st.kb ^ (64 * s)));
        const int4v hi = *(const int4v *)(p + (st.kb ^ (64 * s + 16)));
        return int8v{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }

    // A operand of O^T for d block i: four transpose reads, keys
    // 16t + 4h + {0,1,2,3,8,9,10,11}
    __device__ __forceinline__ static int8v vfrag(const State &st, const uint8_t *vl, int i)
    {
        typedef __attribute__((address_space(3))) int2v lds_int2v;
        const uint8_t *p = vl + (st.vb ^ (32 * i));
        int2v r[4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
            r[t] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_int2v *)(p + 16 * t * D));
        return int8v{r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
    }

    // Mask keys >= Lk and (causal) keys after the query's position qp.
    // Accumulator a, register r holds key k0 + 32a + 8(r/4) + 4h + r%4.
    __device__ __forceinline__ static void mask(floatx16 (&sc)[2], int k0, int Lk, int qp)
    {
        const int h = (threadIdx.x & 63) >> 5;
        int bound = Lk - k0 - 4 * h;
        if (CAUSAL) {
            const int cb = qp - k0 - 4 * h + 1;
            bound = cb < bound ? cb : bound;
        }
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (32 * a + 8 * (r >> 2) + (r & 3) >= bound) sc[a][r] = -__builtin_huge_valf();
    }

    __device__ __forceinline__ static float block_max(const floatx16 (&sc)[2])
    {
        float m0 = fmaxf(fmaxf(sc[0][0], sc[0][1]), sc[0][2]);
        float m1 = fmaxf(fmaxf(sc[1][0], sc[1][1]), sc[1][2]);
#pragma unroll
        for (int r = 3; r < 15; r += 2) {
            m0 = fmaxf(fmaxf(m0, sc[0][r]), sc[0][r + 1]);
            m1 = fmaxf(fmaxf(m1, sc[1][r]), sc[1][r + 1]);
        }
        m0 = fmaxf(fmaxf(m0, sc[0][15]), sc[1][15]);
        return pair_max(fmaxf(m0, m1));
    }

    // Raise the reference maximum to at least mx and rescale O and l; a lane
    // whose maximum does not change keeps factor 1 (never -inf - -inf).
    __device__ __forceinline__ static void raise_to(State &st, float mx, float c)
    {
        const float m_new = fmaxf(st.m, mx);
        const float sf = st.m == m_new ? 1.0f : exp2_fast((st.m - m_new) * c);
        st.l *= sf;
#pragma unroll
        for (int i = 0; i < kDBlocks; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) st.oacc[i][r] *= sf;
        st.m = m_new;
        st.mc = (m_new == -__builtin_huge_valf() ? 0.0f : m_new * c) - kOffsetLog2;
    }

    // 2^3 * P for score pair p (accumulator p/8, registers 2(p%8), +1):
    // E4M3 bytes 16(p/8) + 2(p%8), +1 of the B operand; both fp32 values go
    // into the lane's two partial row sums.
    template <int p>
    __device__ __forceinline__ static void exp_pair(const floatx16 (&sc)[2], int8v &pf, float (&rs)[2],
                                                    float mc, float c)
    {
        constexpr int a = p >> 3, pp = p & 7, r = 2 * pp, w = 4 * a + (pp >> 1);
        const float p0 = exp2_fast(__builtin_fmaf(sc[a][r], c, -mc));
        const float p1 = exp2_fast(__builtin_fmaf(sc[a][r + 1], c, -mc));
        rs[0] += p0;
        rs[1] += p1;
        if constexpr ((pp & 1) == 0)
            pf[w] = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
        else
            pf[w] = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, pf[w], true);
        // keep the pair where it stands in the schedule
        __asm__ volatile("" ::"v"(pf[w]), "v"(rs[0]), "v"(rs[1]));
    }

    template <int P0, int N>
    __device__ __forceinline__ static void exp_pairs(const floatx16 (&sc)[2], int8v &pf, float (&rs)[2],
                                                     float mc, float c)
    {
        if constexpr (N > 0) {
            exp_pair<P0>(sc, pf, rs, mc, c);
            exp_pairs<P0 + 1, N - 1>(sc, pf, rs, mc, c);
        }
    }

    // S^T of one 64-key block, nothing in between
    __device__ __forceinline__ static void s_product(floatx16 (&sc)[2], const State &st, const uint8_t *kl)
    {
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            sc[a] = floatx16{};
#pragma unroll
            for (int s = 0; s < kS; ++s)
                sc[a] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kfrag(st, kl, a, s), st.qf[s],
                                                                         sc[a], 0, 0, 0, 0, 0, 0);
        }
    }

    // MFMA n of the S product of the next block (half n / kS, k-step
    // n % kS), the next MFMA's K operand read ahead, then this MFMA's share
    // of the current block's exponential pairs.
    template <int n>
    __device__ __forceinline__ static void s_with_exps(const State &st, const floatx16 (&sc)[2],
                                                       floatx16 (&sn)[2], int8v &ka, const uint8_t *kl,
                                                       int8v &pf, float (&rs)[2], float mc, float c)
    {
        if constexpr (n < 2 * kS) {
            constexpr int kPer = 16 / (2 * kS);
            int8v kn = ka;
            if constexpr (n + 1 < 2 * kS) kn = kfrag(st, kl, (n + 1) / kS, (n + 1) % kS);
            sn[n / kS] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, st.qf[n % kS], sn[n / kS], 0,
                                                                          0, 0, 0, 0, 0);
            ka = kn;
            exp_pairs<n * kPer, kPer>(sc, pf, rs, mc, c);
            __builtin_amdgcn_sched_barrier(0);
            s_with_exps<n + 1>(st, sc, sn, ka, kl, pf, rs, mc, c);
        }
    }

    // The block's probabilities overran the E4M3 range in some lane: raise
    // the reference to the block's maximum and compute them again.
    __device__ __forceinline__ static void fixup(State &st, const floatx16 (&sc)[2], int8v &pf,
                                                 float (&rs)[2], float c)
    {
        raise_to(st, block_max(sc), c);
        rs[0] = 0.0f;
        rs[1] = 0.0f;
        exp_pairs<0, 16>(sc, pf, rs, st.mc, c);
    }

    // One step for score block u (scores sc complete): MASK it if needed;
    // with NEXT, the S product of block u+1 (into sn, K tile kl) runs with
    // the 16 exponential pairs of block u between its MFMAs; then the
    // overrun test, and the P.V product of block u (V tile vl).
    template <bool NEXT, bool MASK>
    __device__ __forceinline__ static void step(State &st, floatx16 (&sc)[2], floatx16 (&sn)[2],
                                                const uint8_t *kl, const uint8_t *vl, int k0, int Lk,
                                                int qp, float c)
    {
        if constexpr (MASK) mask(sc, k0, Lk, qp);
        // issue priority up for the exponential phase, down for P.V, so the
        // other wavefront of the SIMD feeds the matrix unit meanwhile
        __builtin_amdgcn_s_setprio(1);
        int8v pf;
        float rs[2] = {0.0f, 0.0f};
        const float mc = st.mc;
        if constexpr (NEXT) {
            int8v ka = kfrag(st, kl, 0, 0);
            sn[0] = floatx16{};
            sn[1] = floatx16{};
            s_with_exps<0>(st, sc, sn, ka, kl, pf, rs, mc, c);
        } else {
            exp_pairs<0, 16>(sc, pf, rs, mc, c);
        }
        int8v va = vfrag(st, vl, 0);
        if (__builtin_amdgcn_ballot_w64(rs[0] + rs[1] >= kE4M3Max)) fixup(st, sc, pf, rs, c);
        st.l += rs[0] + rs[1];
        __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int i = 0; i < kDBlocks; ++i) {
            int8v vn = va;
            if (i + 1 < kDBlocks) vn = vfrag(st, vl, i + 1);
            st.oacc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pf, st.oacc[i], 0, 0, 0, 0,
                                                                          0, 0);
            va = vn;
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // Step u with LDS parity P = u % 2: after the barrier, K(u+2) goes to
    // kbuf[P] (K(u) was last read by step u-1) and V(u+1) to vbuf[P^1]
    // (V(u-1) likewise); S(u+1) reads kbuf[P^1], P.V(u) reads vbuf[P].
    template <int P, bool NEXT, bool MASK>
    __device__ __forceinline__ static void block(State &st, floatx16 (&sc)[2], floatx16 (&sn)[2],
                                                 const uint32_t (&offs)[G::kLoadsPerWave],
                                                 const uint8_t *kbase, const uint8_t *vbase,
                                                 int64_t kv_row, int u, int n_blocks, int Lk, int qp,
                                                 float c, uint8_t (*klds)[G::kTile],
                                                 uint8_t (*vlds)[G::kTile])
    {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (u + 2 < n_blocks) issue_tile8_at<D, W>(offs, kbase, kv_row, u + 2, Lk, klds[P]);
        if (u + 1 < n_blocks) issue_tile8_at<D, W>(offs, vbase, kv_row, u + 1, Lk, vlds[P ^ 1]);
        step<NEXT, MASK>(st, sc, sn, klds[P ^ 1], vlds[P], kBlk * u, Lk, qp, c);
    }

    __device__ static void run(const Args8 &a)
    {
        __shared__ __attribute__((aligned(16))) uint8_t klds[2][G::kTile];
        __shared__ __attribute__((aligned(16))) uint8_t vlds[2][G::kTile];

        const int lane = threadIdx.x & 63;
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const int col = lane & 31, h = lane >> 5;

        const int item = xcd_item(blockIdx.x, a.n_items);
        int rest = item / a.n_qblocks;
        int qb = item % a.n_qblocks;
        if (CAUSAL) qb = a.n_qblocks - 1 - qb;  // heaviest blocks first
        const int g = rest % a.groups;
        rest /= a.groups;
        const int hk = rest % a.Hkv;
        const int b = rest / a.Hkv;
        const int hq = hk * a.groups + g;
        const int Lq = a.Lq, Lk = a.Lk;
        const int q0 = qb * kBM;

        const int64_t q_row = (int64_t)a.H * D, kv_row = (int64_t)a.Hkv * D;  // bytes
        const uint8_t *qbase = a.q + (int64_t)b * Lq * q_row + (int64_t)hq * D;
        const uint8_t *kbase = a.k + (int64_t)b * Lk * kv_row + (int64_t)hk * D;
        const uint8_t *vbase = a.v + (int64_t)b * Lk * kv_row + (int64_t)hk * D;

        int kv_end = Lk;
        if (CAUSAL) {
            const int last = (q0 + kBM < Lq ? q0 + kBM : Lq) - 1 + a.past_len;
            kv_end = last < Lk - 1 ? last + 1 : Lk;
        }
        const int n_blocks = kv_end > 0 ? (kv_end + kBlk - 1) / kBlk : 0;

        State st;
        init(st);
        const int qi = q0 + 32 * wave + col;
        const int qp = (qi < Lq ? qi : Lq - 1) + a.past_len;

        if (n_blocks > 0) {
            uint32_t offs[G::kLoadsPerWave];
            {
                const int pc = lane % G::kChunks;
#pragma unroll
                for (int n = 0; n < G::kLoadsPerWave; ++n) {
                    const int row = load_row8<D, W>(wave, n);
                    offs[n] = (uint32_t)(row * kv_row + 16 * (pc ^ f8_swz<D>(row)));
                }
            }
            issue_tile8_at<D, W>(offs, kbase, kv_row, 0, Lk, klds[0]);
            issue_tile8_at<D, W>(offs, vbase, kv_row, 0, Lk, vlds[0]);
#pragma unroll
            for (int s = 0; s < kS; ++s) {
                int8v val = {};
                if (qi < Lq) {
                    const uint8_t *p = qbase + (int64_t)qi * q_row + 64 * s + 32 * h;
                    const int4v lo = *(const int4v *)p;
                    const int4v hi = *(const int4v *)(p + 16);
                    val = int8v{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                }
                st.qf[s] = val;
            }
            const float c = a.c;

            // prologue: S of block 0 and its exact row maximum; K(1) in flight
            floatx16 sa[2], sb[2];
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (n_blocks > 1) issue_tile8_at<D, W>(offs, kbase, kv_row, 1, Lk, klds[1]);
            s_product(sa, st, klds[0]);
            mask(sa, 0, Lk, qp);
            raise_to(st, block_max(sa), c);

            // Blocks u < n_clean need no mask on any wavefront: every key is
            // < Lk and (causal) at or before the work item's first query.
            const int n_main = n_blocks - 1;  // steps with a successor
            int n_clean = Lk / kBlk;
            if (CAUSAL) {
                const int first = q0 + a.past_len;
                const int nc = first < 0 ? 0 : (first + 1) / kBlk;
                n_clean = nc < n_clean ? nc : n_clean;
            }
            const int u_clean = n_clean < n_main ? n_clean : n_main;
            int u = 0;
            for (; u + 1 < u_clean; u += 2) {
                block<0, true, false>(st, sa, sb, offs, kbase, vbase, kv_row, u, n_blocks, Lk, qp, c, klds, vlds);
                block<1, true, false>(st, sb, sa, offs, kbase, vbase, kv_row, u + 1, n_blocks, Lk, qp, c, klds, vlds);
            }
            if (u < u_clean) {
                block<0, true, false>(st, sa, sb, offs, kbase, vbase, kv_row, u, n_blocks, Lk, qp, c, klds, vlds);
                ++u;
                if (u < n_main) {
                    block<1, true, true>(st, sb, sa, offs, kbase, vbase, kv_row, u, n_blocks, Lk, qp, c, klds, vlds);
                    ++u;
                }
            }
            // from here u is even whenever the scores of block u are in sa
            if (u & 1) {
                // only reached with u == n_main (odd): last block's scores in sb
                if (n_blocks > n_clean)
                    block<1, false, true>(st, sb, sa, offs, kbase, vbase, kv_row, u, n_blocks, Lk, qp, c, klds, vlds);
                else
                    block<1, false, false>(st, sb, sa, offs, kbase, vbase, kv_row, u, n_blocks, Lk, qp, c, klds, vlds);
            } else {
                for (; u + 1 < n_main; u += 2) {
                    block<0, true, true>(st, sa, sb, offs, kbase, vbase, kv_row, u, n_blocks, Lk, qp, c, klds, vlds);
                    block<1, true, true>(st, sb, sa, offs, kbase, vbase, kv_row, u + 1, n_blocks, Lk, qp, c, klds, vlds);
                }
                if (u < n_main) {
                    block<0, true, true>(st, sa, sb, offs, kbase, vbase, kv_row, u, n_blocks, Lk, qp, c, klds, vlds);
                    ++u;
                    if (n_blocks > n_clean)
                        block<1, false, true>(st, sb, sa, offs, kbase, vbase, kv_row, u, n_blocks, Lk, qp, c, klds, vlds);
                    else
                        block<1, false, false>(st, sb, sa, offs, kbase, vbase, kv_row, u, n_blocks, Lk, qp, c, klds, vlds);
                } else {
                    if (n_blocks > n_clean)
                        block<0, false, true>(st, sa, sb, offs, kbase, vbase, kv_row, u, n_blocks, Lk, qp, c, klds, vlds);
                    else
                        block<0, false, false>(st, sa, sb, offs, kbase, vbase, kv_row, u, n_blocks, Lk, qp, c, klds, vlds);
                }
            }
        }

        // O = v_descale * acc / l (guarded as on the page); LSE = scale' * m + ln(l / 2^3)
        const float lt = pair_sum(st.l);
        const float inv = a.v_descale / (lt > 1e-6f ? lt : 1.0f);
        // Register 4rb+J of d block i holds d = 32i + 8rb + 4h + J.  For each
        // pair rb = 2e, 2e+1 the lane halves swap one packed pair
        // (v_permlane32_swap: the upper lanes of the first operand trade with
        // the lower lanes of the second); then half 0 holds d = 32i+16e+0..7
        // and half 1 d = 32i+16e+8..15, so every lane stores 16 contiguous
        // bytes of its row.  Lanes l and l^32 share a row: every lane takes
        // part in the exchange.
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
            _Float16 *orow = a.o + ((int64_t)b * Lq + qi) * a.H * D + (int64_t)hq * D;
#pragma unroll
            for (int i = 0; i < kDBlocks; ++i)
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const uint4v v4 = {ow[i][e][0], ow[i][e][1], ow[i][e][2], ow[i][e][3]};
                    *(uint4v *)(orow + 32 * i + 16 * e + 8 * h) = v4;
                }
            if (a.lse && h == 0)
                a.lse[((int64_t)b * a.H + hq) * Lq + qi] = st.m * a.lse_scale + __logf(lt) - kOffsetLog2 * kLn2;
        }
    }
};

template <int D, bool CAUSAL, int W>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * W, 64 * W),
                          amdgpu_waves_per_eu(2, 2))) void
fa_fwd_fp8_kernel(const Args8 a)
{
    Kernel8<D, CAUSAL, W>::run(a);
}

template <int D, bool CAUSAL>
int launch8(Args8 args, hipStream_t stream)
{
    constexpr int W = CAUSAL ? 4 : 8;
    using K = Kernel8<D, CAUSAL, W>;
    args.n_qblocks = (args.Lq + K::kBM - 1) / K::kBM;
    const int64_t items = (int64_t)args.n_items * args.n_qblocks;  // n_items holds B*H here
    if (items > 0x7fffffff) return FA_ERR_SHAPE;
    args.n_items = (int)items;
    hipLaunchKernelGGL((fa_fwd_fp8_kernel<D, CAUSAL, W>), dim3(args.n_items), dim3(K::kThreads), 0,
                       stream, args);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

int launch_forward_fp8(const Problem &p, Fp8Descale ds, hipStream_t stream)
{
    // per-lane tile offsets are 32-bit: a tile of kBlk K/V rows must span < 2 GiB
    if ((int64_t)p.Hkv * p.D * kBlk > 0x7fffffff) return FA_ERR_SHAPE;
    const int64_t bh = (int64_t)p.B * p.H;
    if (bh > 0x7fffffff) return FA_ERR_SHAPE;
    Args8 a;
    a.q = (const uint8_t *)p.q;
    a.k = (const uint8_t *)p.k;
    a.v = (const uint8_t *)p.v;
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
    a.lse_scale = p.scale * ds.q * ds.k;
    a.c = a.lse_scale * 1.4426950408889634f;
    a.v_descale = ds.v;
    if (p.D == 64) return p.causal ? launch8<64, true>(a, stream) : launch8<64, false>(a, stream);
    return p.causal ? launch8<128, true>(a, stream) : launch8<128, false>(a, stream);
}

}  // namespace fa
