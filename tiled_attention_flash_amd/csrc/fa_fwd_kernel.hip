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
// * Workgroup = 4 wavefronts (256 lanes) owning one block of BM = 128 query
//   rows of one (batch, query head); each wavefront owns 32 whole query rows.
// * Both products are computed transposed, on v_mfma_f32_32x32x16_f16:
//     S^T[key][query]  = K . Q^T     (A = K rows from LDS, B = Q from VGPRs)
//     O^T[d][query]   += V^T . P^T   (A = V^T from LDS,    B = P from VGPRs)
//   In the 32x32 accumulator layout lane l holds column l%32, i.e. one query,
//   and 16 of its 32 rows (keys, or d) -- the other 16 live in lane l^32.
//   Row statistics are therefore per-lane values plus ONE exchange between
//   the two 32-lane halves (v_permlane32_swap), and the per-row rescale of
//   O^T is a per-lane scalar.
// * The S^T accumulator registers, converted to fp16, are exactly the B
//   operand of the second product once the 16 keys of each k-step are taken
//   in the order the accumulator holds them; V^T is stored in LDS in that
//   same key order, so P never leaves registers.
// * K/V tiles of BN = 64 keys: 128-bit coalesced global loads into registers
//   one tile ahead, then stored to a double-buffered LDS tile (K row-major
//   with a 16-byte row pad, V transposed with an XOR-swizzled 16-byte chunk
//   order) -- one workgroup barrier per tile.
// * Causal: tiles past the block's last query are never visited; the mask
//   code runs only on tiles that straddle a wavefront's diagonal (or hold
//   the ragged end of the sequence).
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
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;  // query rows per work item
constexpr int kBN = 64;           // keys per K/V tile
constexpr int kXcds = 8;

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
// own value in one result and lane l^32's value in the other.  Combining the
// two symmetrically gives the cross-half max / sum without caring which is
// which.
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

// Position, inside a tile of kBN keys, at which V^T stores key `key` so that
// a 16-byte LDS read returns the 8 keys lane-half `h` of the k-step needs:
// k-step c covers keys 16c..16c+15; the accumulator holds, for lane half h,
// keys 16c + {4h..4h+3, 8+4h..8+4h+3} in that order.
__device__ __forceinline__ int vt_position(int key)
{
    int c = key >> 4, r = key & 15;
    int a = r >> 3, h = (r >> 2) & 1, j = r & 3;
    return 16 * c + 8 * h + 4 * a + j;
}

// 16-byte chunk swizzle of V^T rows (kBN = 64 halves = 8 chunks per row): a
// 16-byte read by 16 consecutive rows, and by 8 consecutive rows, touches
// every LDS bank exactly once.
__device__ __forceinline__ int vt_chunk(int d, int chunk) { return chunk ^ ((d + (d >> 3)) & 7); }

template <int D>
struct Tiles {
    static constexpr int kKStride = D + 8;            // halves per K row in LDS (16-byte pad)
    static constexpr int kKTile = kBN * kKStride;     // halves
    static constexpr int kVTile = D * kBN;            // halves
    static constexpr int kKUnits = kBN * D / 8;       // 16-byte K chunks per tile
    static constexpr int kKPerThread = kKUnits / kThreads;
    static constexpr int kDGroups = D / 8;
    static constexpr int kVUnits = (kBN / 4) * kDGroups;  // (4 keys x 8 d) blocks per tile
    static constexpr int kVPerThread = (kVUnits + kThreads - 1) / kThreads;
    static_assert(kKUnits % kThreads == 0, "K tile must split evenly");
};

template <int D>
struct Prefetch {
    u32x4 k[Tiles<D>::kKPerThread];
    u32x4 v[Tiles<D>::kVPerThread][4];
};

// Global -> registers for the K/V tile starting at key k0.  Rows at or past
// L are zero-filled so masked keys carry finite values.
template <int D>
__device__ __forceinline__ void load_tile(Prefetch<D> &pf, const _Float16 *kbase,
                                          const _Float16 *vbase, int64_t kv_row, int k0, int L)
{
    using T = Tiles<D>;
    const int tid = threadIdx.x;
#pragma unroll
    for (int r = 0; r < T::kKPerThread; ++r) {
        int u = tid + r * kThreads;
        int row = u / T::kDGroups, ch = u % T::kDGroups;
        int key = k0 + row;
        u32x4 val = {0, 0, 0, 0};
        if (key < L) val = *(const u32x4 *)(kbase + (int64_t)key * kv_row + ch * 8);
        pf.k[r] = val;
    }
#pragma unroll
    for (int r = 0; r < T::kVPerThread; ++r) {
        int u = tid + r * kThreads;
        // u = kg_hi * (4 * kDGroups) + dg * 4 + kg_lo, kg = 4 * kg_hi + kg_lo
        int kg = 4 * (u / (4 * T::kDGroups)) + (u & 3);
        int dg = (u >> 2) % T::kDGroups;
        bool active = u < T::kVUnits;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int key = k0 + 4 * kg + j;
            u32x4 val = {0, 0, 0, 0};
            if (active && key < L) val = *(const u32x4 *)(vbase + (int64_t)key * kv_row + dg * 8);
            pf.v[r][j] = val;
        }
    }
}

// Registers -> LDS: K row-major (padded), V transposed into V^T[d][position].
template <int D>
__device__ __forceinline__ void store_tile(const Prefetch<D> &pf, _Float16 *klds, _Float16 *vlds)
{
    using T = Tiles<D>;
    const int tid = threadIdx.x;
#pragma unroll
    for (int r = 0; r < T::kKPerThread; ++r) {
        int u = tid + r * kThreads;
        int row = u / T::kDGroups, ch = u % T::kDGroups;
        *(u32x4 *)(klds + row * T::kKStride + ch * 8) = pf.k[r];
    }
#pragma unroll
    for (int r = 0; r < T::kVPerThread; ++r) {
        int u = tid + r * kThreads;
        if (u >= T::kVUnits) continue;
        int kg = 4 * (u / (4 * T::kDGroups)) + (u & 3);
        int dg = (u >> 2) % T::kDGroups;
        int pos = vt_position(4 * kg);  // the 4 keys stay contiguous
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            int w = e >> 1;
            uint32_t a0 = pf.v[r][0][w], a1 = pf.v[r][1][w], a2 = pf.v[r][2][w], a3 = pf.v[r][3][w];
            u32x2 out;
            if (e & 1) {
                out[0] = (a0 >> 16) | (a1 & 0xffff0000u);
                out[1] = (a2 >> 16) | (a3 & 0xffff0000u);
            } else {
                out[0] = (a0 & 0xffffu) | (a1 << 16);
                out[1] = (a2 & 0xffffu) | (a3 << 16);
            }
            int d = 8 * dg + e;
            int off = d * kBN + 8 * vt_chunk(d, pos >> 3) + (pos & 7);
            *(u32x2 *)(vlds + off) = out;
        }
    }
}

// Work item -> (b, kv head, group member, q block).  Items are ordered so
// that the query heads sharing one K/V head, and all q blocks of each, are
// consecutive.
__device__ __forceinline__ int xcd_item(int block, int n)
{
    int x = block % kXcds, slot = block / kXcds;
    int per = n / kXcds, extra = n % kXcds;
    return x * per + (x < extra ? x : extra) + slot;
}

template <int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(2, 2))) void
fa_fwd_kernel(const Args a)
{
    using T = Tiles<D>;
    constexpr int kSteps = D / 16;   // k-steps of S^T = K.Q^T
    constexpr int kDBlocks = D / 32; // 32-row blocks of O^T
    __shared__ __attribute__((aligned(16))) _Float16 klds[2][T::kKTile];
    __shared__ __attribute__((aligned(16))) _Float16 vlds[2][T::kVTile];

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

    // ---- Q block -> B-operand fragments (lane: query q0 + 32*wave + col)
    const int wq0 = q0 + 32 * wave;
    const int qi = wq0 + col;
    half8 qf[kSteps];
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        half8 val = {};
        if (qi < L) val = *(const half8 *)(qbase + (int64_t)qi * q_row + 16 * s + 8 * half);
        qf[s] = val;
    }

    floatx16 oacc[kDBlocks];
#pragma unroll
    for (int i = 0; i < kDBlocks; ++i) oacc[i] = floatx16{};
    float m = -__builtin_huge_valf();  // running row max (raw score units)
    float l = 0.0f;                    // running row sum (this lane's keys)

    const int kv_end = CAUSAL ? (q0 + kBM < L ? q0 + kBM : L) : L;
    const int n_tiles = (kv_end + kBN - 1) / kBN;
    const float c = a.scale_log2;

    Prefetch<D> pf;
    load_tile<D>(pf, kbase, vbase, kv_row, 0, L);
    store_tile<D>(pf, klds[0], vlds[0]);

    for (int t = 0; t < n_tiles; ++t) {
        const int k0 = t * kBN;
        const bool more = t + 1 < n_tiles;
        if (more) load_tile<D>(pf, kbase, vbase, kv_row, k0 + kBN, L);
        __syncthreads();
        const _Float16 *kl = klds[t & 1];
        const _Float16 *vl = vlds[t & 1];

        // A wavefront whose 32 queries all precede this tile has nothing to do.
        const bool active = !CAUSAL || k0 <= wq0 + 31;
        if (active) {
            // S^T = K . Q^T for the 64 keys of the tile, as two 32-key blocks
            floatx16 sacc[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                floatx16 acc = {};
#pragma unroll
                for (int s = 0; s < kSteps; ++s) {
                    half8 ka = *(const half8 *)(kl + (32 * kb + col) * T::kKStride + 16 * s + 8 * half);
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka, qf[s], acc, 0, 0, 0);
                }
                sacc[kb] = acc;
            }

            // mask: keys past the sequence end, and keys after the query (causal)
            const bool need_mask = (k0 + kBN > L) || (CAUSAL && k0 + kBN - 1 > wq0);
            if (need_mask) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * half + (r & 3);
                        bool hide = key >= L || (CAUSAL && key > qi);
                        if (hide) sacc[kb][r] = -__builtin_huge_valf();
                    }
            }

            // online softmax (exp via exp2 with scale*log2(e) folded in)
            float mx = sacc[0][0];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
            mx = pair_max(mx);
            const float m_new = fmaxf(m, mx);
            const float mc = m_new * c;
            const float sf = exp2_fast(m * c - mc);
            float rs = 0.0f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float p = exp2_fast(__builtin_fmaf(sacc[kb][r], c, -mc));
                    sacc[kb][r] = p;
                    rs += p;
                }
            l = l * sf + rs;
            m = m_new;
#pragma unroll
            for (int i = 0; i < kDBlocks; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[i][r] *= sf;

            // P^T k-steps (16 keys each) as fp16 B operands, round-to-nearest-even
            half8 pfrag[4];
#pragma unroll
            for (int cs = 0; cs < 4; ++cs) {
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    float2v f2 = {sacc[cs >> 1][8 * (cs & 1) + e], sacc[cs >> 1][8 * (cs & 1) + e + 1]};
                    half2v h2 = __builtin_convertvector(f2, half2v);
                    pfrag[cs][e] = h2[0];
                    pfrag[cs][e + 1] = h2[1];
                }
            }

            // O^T += V^T . P^T
#pragma unroll
            for (int i = 0; i < kDBlocks; ++i) {
                const int d = 32 * i + col;
#pragma unroll
                for (int cs = 0; cs < 4; ++cs) {
                    half8 va = *(const half8 *)(vl + d * kBN + 8 * vt_chunk(d, 2 * cs + half));
                    oacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pfrag[cs], oacc[i], 0, 0, 0);
                }
            }
        }

        if (more) store_tile<D>(pf, klds[(t + 1) & 1], vlds[(t + 1) & 1]);
    }

    // ---- finalise: O = acc / l (guarded as on the page), LSE = scale*m + ln l
    const float lt = pair_sum(l);
    const float inv = 1.0f / (lt > 1e-6f ? lt : 1.0f);
    if (qi < L) {
        _Float16 *orow = a.o + (int64_t)b * L * q_row + (int64_t)qi * q_row + (int64_t)h * D;
#pragma unroll
        for (int i = 0; i < kDBlocks; ++i)
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                float2v lo = {oacc[i][4 * rb + 0] * inv, oacc[i][4 * rb + 1] * inv};
                float2v hi = {oacc[i][4 * rb + 2] * inv, oacc[i][4 * rb + 3] * inv};
                half2v hl = __builtin_convertvector(lo, half2v);
                half2v hh = __builtin_convertvector(hi, half2v);
                half4 out = {hl[0], hl[1], hh[0], hh[1]};
                *(half4 *)(orow + 32 * i + 8 * rb + 4 * half) = out;
            }
        if (a.lse && half == 0)
            a.lse[((int64_t)b * a.H + h) * L + qi] = m * a.scale + __logf(lt);
    }
}

template <int D, bool CAUSAL>
int launch(const Args &args, hipStream_t stream)
{
    hipLaunchKernelGGL((fa_fwd_kernel<D, CAUSAL>), dim3(args.n_items), dim3(kThreads), 0, stream,
                       args);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

int launch_forward(const Problem &p, hipStream_t stream)
{
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
    a.n_qblocks = (p.L + kBM - 1) / kBM;
    int64_t items = (int64_t)p.B * p.H * a.n_qblocks;
    if (items > 0x7fffffff) return FA_ERR_SHAPE;
    a.n_items = (int)items;
    a.scale = p.scale;
    a.scale_log2 = p.scale * 1.4426950408889634f;
    if (p.D == 64) return p.causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
    return p.causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
}

}  // namespace fa
