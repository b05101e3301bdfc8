// fa_device.h -- device code shared by the attention kernels (gfx950): operand
// types, cross-lane helpers, LDS swizzles, direct HBM -> LDS loads, and the
// per-wavefront arithmetic of one 32-key score block -- the MFMA operand
// reads, the mask, the row maximum, the lazy rescale and the exponentials.
//
// Method: page "使用 TileLang 在 AMD GPU 上快速开发高性能 Flash Attention",
// section "K/V Tile 遍历与核心计算" (Q K^T, mask, row max, rescale, exp, row
// sum, P cast to fp16, P V).
//
// A wavefront owns 32 query rows.  Both products run transposed on
// v_mfma_f32_32x32x16_f16:
//   S^T[key][row]  = K . Q^T     (A = K rows from LDS, B = Q in VGPRs)
//   O^T[d][row]   += V^T . P^T   (A = V^T from LDS,   B = P in VGPRs)
// In the 32x32 accumulator layout lane l holds column l%32 -- one query row
// -- and 16 of its 32 rows (keys, or d); the other 16 live in lane l^32.  So
// row statistics are per-lane values plus one exchange between the two
// 32-lane halves, and the rescale of O^T is a per-lane scalar.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t uint4v __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))

constexpr int kSB = 32;               // keys per score block (one 32x32 accumulator)
constexpr int kXcds = 8;
constexpr float kRescaleLog2 = 8.0f;  // lazy-rescale threshold (exp2 domain)
// A lane's sum of the (fp32) probabilities of one score block at or above
// which the block is recomputed against its own maximum.  Every kept
// probability is then below 2^15, far from fp16's largest finite value
// (65504), and a probability that would round to inf in fp16, or is inf in
// fp32, always fails the test.
constexpr float kSumLimit = 32768.0f;

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

// One 16-byte-per-lane direct HBM -> LDS load: lane i's 16 bytes from
// base + off land at lds + 16*i.  Written as inline assembly so that the
// compiler does not see the LDS tile buffers as written by an in-flight load
// and stall every later LDS read until all loads complete (it cannot tell
// the buffers apart); the kernels wait for a tile's loads themselves.
__device__ __forceinline__ void dma16(const char *base, uint32_t off, _Float16 *lds)
{
    const uint32_t m0 = (uint32_t)(uintptr_t)(LDS_AS void *)lds;
    __asm__ volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                     :
                     : "v"(off), "s"(base), "{m0}"(m0)
                     : "memory");
}

__device__ __forceinline__ half8 lds_read16(const _Float16 *p) { return *(const half8 *)p; }

__device__ __forceinline__ half4 lds_read_tr(const _Float16 *p)
{
    short4v v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS short4v *)(p));
    return __builtin_bit_cast(half4, v);
}

// Workgroup id -> work item, so that each of the 8 XCDs (which receive
// workgroups round-robin) walks a contiguous range of the n work items.
__device__ __forceinline__ int xcd_item(int block, int n)
{
    int x = block % kXcds, slot = block / kXcds;
    int per = n / kXcds, extra = n % kXcds;
    return x * per + (x < extra ? x : extra) + slot;
}

// Per-wavefront arithmetic of one 32-key score block, head dim D.
template <int D, bool CAUSAL>
struct WaveMath {
    static constexpr int kSteps = D / 16;    // k-steps of S^T = K.Q^T
    static constexpr int kDBlocks = D / 32;  // 32-row blocks of O^T
    static constexpr int kCS = kSB / 16;     // 16-key k-steps of P.V per score block
    static constexpr int kPairs = 8;         // score pairs per lane per score block

    // per-lane state of one wavefront
    struct State {
        half8 qf[kSteps];
        floatx16 oacc[kDBlocks];
        float m;     // reference row maximum (raw score units)
        float mc;    // m * c, c = scale * log2(e)
        float l;     // running row sum, this lane's keys
        int k_base;  // LDS half offset of this lane's K read at k-step 0
        int v_base;  // LDS half offset of this lane's V transpose read at d block 0
    };

    __device__ __forceinline__ static void init(State &st)
    {
#pragma unroll
        for (int i = 0; i < kDBlocks; ++i) st.oacc[i] = floatx16{};
        st.m = -__builtin_huge_valf();
        st.mc = 0.0f;
        st.l = 0.0f;
    }

    // LDS read bases for K and V tiles stored row-major (D halves per row)
    // with the k_chunk / v_chunk swizzles, row 0 at the block's first key.
    __device__ __forceinline__ static void init_lds_bases(State &st, int lane)
    {
        const int col = lane & 31, half = lane >> 5;
        // K: row = col, logical chunk 2s + half at k-step s
        st.k_base = col * D + 8 * k_chunk<D>(col, half);
        // V transpose read: 16-lane group gg = lane/16 (d half gg%2, key
        // half gg/2), j = lane%16 -> row 4*(gg/2) + j/4 (+ 16*cs [+ 8]),
        // d = 32*i + 16*(gg%2) + 4*(j%4)
        const int gg = lane >> 4, j = lane & 15;
        const int row = 4 * (gg >> 1) + (j >> 2);
        const int d = 16 * (gg & 1) + 4 * (j & 3);
        st.v_base = row * D + 8 * v_chunk<D>(row, d >> 3) + (d & 7);
    }

    // The swizzles are XORs on the 16-byte chunk index, and the chunk index
    // of k-step s (d block i) differs from that of step 0 (block 0) only in
    // bits the XOR touches, so each read address is one XOR from the base.
    __device__ __forceinline__ static int k_offset(const State &st, int s) { return st.k_base ^ (16 * s); }
    __device__ __forceinline__ static int v_offset(const State &st, int i) { return st.v_base ^ (32 * i); }

    // A operand of S^T for k-step s; kl points at the block's first K row
    __device__ __forceinline__ static half8 kfrag(const State &st, const _Float16 *kl, int s)
    {
        return lds_read16(kl + k_offset(st, s));
    }

    // A operand of O^T for d block i and k-step cs; vl points at the block's
    // first V row.  Two transpose reads: keys 16cs + 4h + 0..3 and
    // 16cs + 8 + 4h + 0..3 for lane half h.
    __device__ __forceinline__ static half8 vfrag(const State &st, const _Float16 *vl, int i, int cs)
    {
        const _Float16 *p = vl + v_offset(st, i) + 16 * cs * D;
        const half4 lo = lds_read_tr(p);
        const half4 hi = lds_read_tr(p + 8 * D);
        return half8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }

    // The block at key k0 holds keys past the end of the keys, or (causal)
    // keys after the position wp0 of the wavefront's first query.
    __device__ __forceinline__ static bool needs_mask(int k0, int Lk, int wp0)
    {
        return (k0 + kSB > Lk) || (CAUSAL && k0 + kSB - 1 > wp0);
    }

    // Mask keys past the end of the keys, and (causal) keys after the query's
    // position qp (its row plus past_len).  Register r holds key
    // k0 + h4 + 8(r/4) + r%4 (h4 = 4 * the lane's half), so one per-lane
    // bound decides every element.
    __device__ __forceinline__ static void mask(floatx16 &sacc, int k0, int Lk, int qp, int h4)
    {
        int bound = Lk - k0 - h4;  // hide offsets >= bound
        if (CAUSAL) {
            const int cb = qp - k0 - h4 + 1;
            bound = cb < bound ? cb : bound;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if (8 * (r >> 2) + (r & 3) >= bound) sacc[r] = -__builtin_huge_valf();
    }

    // Row maximum of a score block over both lane halves -- a tree of
    // 3-input maxima, then one cross-half exchange -- in stages that can be
    // spread between other instructions.
    struct MaxTree {
        static constexpr int kStages = 5;
        float a, b, d, e, f, g, h, mx;
        __device__ __forceinline__ void stage(int i, const floatx16 &x)
        {
            switch (i) {
            case 0:
                a = fmaxf(fmaxf(x[0], x[1]), x[2]);
                b = fmaxf(fmaxf(x[3], x[4]), x[5]);
                break;
            case 1:
                d = fmaxf(fmaxf(x[6], x[7]), x[8]);
                e = fmaxf(fmaxf(x[9], x[10]), x[11]);
                break;
            case 2:
                f = fmaxf(fmaxf(x[12], x[13]), x[14]);
                g = fmaxf(fmaxf(a, b), d);
                break;
            case 3: h = fmaxf(fmaxf(e, f), x[15]); break;
            default: mx = pair_max(fmaxf(g, h)); break;
            }
        }
    };

    __device__ __forceinline__ static float block_max(const floatx16 &x)
    {
        MaxTree t;
#pragma unroll
        for (int i = 0; i < MaxTree::kStages; ++i) t.stage(i, x);
        return t.mx;
    }

    // S^T = K . Q^T for one score block, no other work in between
    __device__ __forceinline__ static void s_product(floatx16 &sacc, const State &st, const _Float16 *kl)
    {
        half8 ka[kSteps];
#pragma unroll
        for (int s = 0; s < kSteps; ++s) ka[s] = kfrag(st, kl, s);
        sacc = floatx16{};
#pragma unroll
        for (int s = 0; s < kSteps; ++s)
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[s], st.qf[s], sacc, 0, 0, 0);
    }

    // Lazy rescale: raise the reference maximum only when some row's block
    // maximum outgrew it by more than 2^kRescaleLog2 (decided for the whole
    // wavefront); O and l are scaled by the same factor.  A row that has
    // seen no key yet keeps m = -inf and uses 0 as its exponent offset, so
    // its masked scores still give exp2(-inf) = 0 (never -inf - -inf); its
    // first visible key always takes this branch.
    __device__ __forceinline__ static void rescale(State &st, float mx, float c)
    {
        const bool grow = (mx - st.m) * c > kRescaleLog2;
        if (__builtin_amdgcn_ballot_w64(grow)) {
            const float m_new = fmaxf(st.m, mx);
            const float sf = st.m == m_new ? 1.0f : exp2_fast((st.m - m_new) * c);
            st.l *= sf;
#pragma unroll
            for (int i = 0; i < kDBlocks; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) st.oacc[i][r] *= sf;
            st.m = m_new;
            st.mc = m_new == -__builtin_huge_valf() ? 0.0f : m_new * c;
        }
    }

    // Raise the reference maximum to at least mx (per lane) and rescale O
    // and l to it; a lane whose maximum does not change keeps factor 1.
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
        st.mc = m_new == -__builtin_huge_valf() ? 0.0f : m_new * c;
    }

    // P = exp2(S*c - m*c) for score pair p (registers 2p, 2p+1), rounded to
    // fp16 (round-to-nearest-even) into the B operand of k-step cs = p/4 of
    // the P.V product at position 2(p%4).  The row sum adds the fp32 values,
    // one per partial sum: plain adds run beside the matrix unit, while a
    // v_dot2_f32_f16 over the fp16 values waits for it (measured: about 11
    // cycles each with MFMAs in flight).  The sum differs from that of the
    // fp16 weights by at most one fp16 rounding (2^-11 relative).
    __device__ __forceinline__ static void exp_pair(const floatx16 &sc, half8 (&pf)[kCS], float (&rs)[2],
                                                    int p, float mc, float c)
    {
        const int r = 2 * p, cs = r >> 3, e = r & 7;
        const float p0 = exp2_fast(__builtin_fmaf(sc[r], c, -mc));
        const float p1 = exp2_fast(__builtin_fmaf(sc[r + 1], c, -mc));
        const float2v f2 = {p0, p1};
        const half2v h2 = __builtin_convertvector(f2, half2v);
        rs[0] += p0;
        rs[1] += p1;
        pf[cs][e] = h2[0];
        pf[cs][e + 1] = h2[1];
        // keep the pair where it stands in the schedule: without a use here
        // the compiler sinks it towards its first MFMA
        __asm__ volatile("" ::"v"(h2), "v"(rs[0]), "v"(rs[1]));
    }
};

}  // namespace
}  // namespace fa
