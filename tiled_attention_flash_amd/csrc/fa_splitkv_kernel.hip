// fa_splitkv_kernel.hip -- split-KV attention forward (flash-decoding) for
// gfx950: few query rows against a long key sequence.
//
// Method: the key range is cut into splits that separate workgroups process
// in parallel, each producing a partial output and log-sum-exp over its own
// keys; a second kernel merges the partials (page "TileLang性能分析报告：H100
// 上FlashAttention吞吐量达1.2PFlops", section "生产环境部署建议", item 2,
// names flash decoding; the per-split arithmetic is that of page "使用
// TileLang 在 AMD GPU 上快速开发高性能 Flash Attention", section "K/V Tile
// 遍历与核心计算").  For a split p with keys J_p and a query row:
//   LSE_p = ln sum_{j in J_p} exp(s_j),  O_p = sum_{j in J_p} exp(s_j - LSE_p) V_j
// and since the splits partition the visible keys,
//   LSE = ln sum_p exp(LSE_p),          O = sum_p exp(LSE_p - LSE) O_p,
// which the merge evaluates with the largest LSE_p subtracted first.
//
// Mapping onto CDNA4
// ------------------
// * With few query rows the pass is bound by reading K and V once from HBM,
//   and the matrix unit has far more throughput than it needs.  So one
//   wavefront (one workgroup) per (b, kv head, row block, split): the g query
//   heads that share a K/V head are packed with the query rows into the 32
//   MFMA columns (packed row R = i*g + j for query row i and head j of the
//   group), so every K/V byte loaded serves all of them.
// * Each wavefront streams its split through a private ring of NST stages in
//   LDS, each holding a 32-key K tile and a 32-key V tile filled by
//   global_load_lds_dwordx4 (HBM -> LDS, no staging registers) with the same
//   chunk swizzles as the full forward kernel.  There are no workgroup
//   barriers: the wavefront waits on its own vector-memory counter for the
//   oldest stage while the next NST-1 stages stay in flight.
// * The block arithmetic (S^T = K.Q^T and O^T += V^T.P^T on
//   v_mfma_f32_32x32x16_f16, mask, lazy-rescaled online softmax) is shared
//   with the full forward kernel.
// * Partials go to a caller-provided fp32 workspace, laid out so that the
//   splits of one output row are contiguous: O_p [B][H][Lq][n_splits][D],
//   LSE_p [B][H][Lq][n_splits].  Every split writes its rows, an empty one
//   O_p = 0 and LSE_p = -inf.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

struct SplitArgs {
    const _Float16 *q, *k, *v;
    float *ws_o, *ws_lse;
    int Lq, Lk;
    int past_len;  // position of query row 0 among the keys (causal only)
    int H, Hkv, groups;
    int n_rb;      // 32-row blocks of the Lq*groups packed rows
    int n_splits;
    int n_items;   // B * Hkv * n_rb * n_splits
    int split_blocks;  // 32-key blocks per split
    int kv_vis;        // keys [0, kv_vis) are visible to some query
    float scale, scale_log2;
};

struct MergeArgs {
    const float *ws_o, *ws_lse;
    _Float16 *o;
    float *lse;
    int Lq, H, n_splits;
    int64_t n_rows;  // B * H * Lq
};

// Wait until at most N of this wavefront's vector-memory loads are
// outstanding (loads complete in issue order), leaving the other counters
// unconstrained.  gfx9 s_waitcnt immediate: vmcnt[3:0] in bits 3:0,
// expcnt in 6:4, lgkmcnt in 11:8, vmcnt[5:4] in 15:14.  The builtin (not
// inline assembly) lets the compiler's own wait insertion see it -- it
// would otherwise keep the Q loads pending and drain the ring every
// iteration; the empty assembly statement with a memory clobber after it
// keeps the LDS reads of the awaited stage below the wait (the compiler
// does not know that the direct loads write LDS).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
    __asm__ volatile("" ::: "memory");
}

template <int D, bool CAUSAL, int NST>
struct SplitKernel : WaveMath<D, CAUSAL> {
    using M = WaveMath<D, CAUSAL>;
    using typename M::State;
    static constexpr int kChunks = D / 8;              // 16-byte chunks per row
    static constexpr int kRowsPerLoad = 64 / kChunks;  // rows one wave load instruction fills
    static constexpr int kLoads = kSB / kRowsPerLoad;  // load instructions per 32-row tile
    static constexpr int kTile = kSB * D;              // halves per K (or V) tile
    static constexpr int kStageLoads = 2 * kLoads;     // K and V tile of one stage
    static_assert(NST >= 2 && (NST - 1) * kStageLoads < 64, "ring too deep for vmcnt");

    // Byte offsets, relative to a tile's first key row, of the 16-byte chunks
    // this lane copies with each load instruction; the swizzle is applied on
    // the source side so that the chunks land in LDS in swizzled order.
    struct Loads {
        uint32_t k[kLoads], v[kLoads];
    };

    __device__ __forceinline__ static int load_row(int n) { return kRowsPerLoad * n + (int)threadIdx.x / kChunks; }

    __device__ __forceinline__ static void init_loads(Loads &lo, int64_t kv_row)
    {
        const int pc = (int)threadIdx.x % kChunks;
#pragma unroll
        for (int n = 0; n < kLoads; ++n) {
            const int row = load_row(n);
            lo.k[n] = (uint32_t)(2 * (row * kv_row + 8 * k_chunk<D>(row, pc)));
            lo.v[n] = (uint32_t)(2 * (row * kv_row + 8 * v_chunk<D>(row, pc)));
        }
    }

    // Issue the K and V loads of the 32-key tile starting at key k0 (>= 0)
    // into one ring stage.  Rows at or past Lk load row Lk-1 instead (finite
    // data that the mask hides).
    __device__ __forceinline__ static void issue_stage(const Loads &lo, const _Float16 *kbase,
                                                       const _Float16 *vbase, int64_t kv_row, int k0,
                                                       int Lk, _Float16 *kl, _Float16 *vl)
    {
        const char *kt = (const char *)(kbase + (int64_t)k0 * kv_row);
        const char *vt = (const char *)(vbase + (int64_t)k0 * kv_row);
        const bool full = k0 + kSB <= Lk;
#pragma unroll
        for (int n = 0; n < kLoads; ++n) {
            uint32_t back = 0;
            if (!full) {
                const int over = k0 + load_row(n) - (Lk - 1);
                if (over > 0) back = (uint32_t)(2 * over * kv_row);
            }
            dma16(kt, lo.k[n] - back, kl + 512 * n);
        }
#pragma unroll
        for (int n = 0; n < kLoads; ++n) {
            uint32_t back = 0;
            if (!full) {
                const int over = k0 + load_row(n) - (Lk - 1);
                if (over > 0) back = (uint32_t)(2 * over * kv_row);
            }
            dma16(vt, lo.v[n] - back, vl + 512 * n);
        }
    }

    // Wait for the stage of block t when `ahead` later stages are in flight
    // (0 <= ahead <= NST-1).
    __device__ __forceinline__ static void wait_stage(int ahead)
    {
        if (ahead >= NST - 1) {
            wait_vmcnt<(NST - 1) * kStageLoads>();
            return;
        }
        switch (ahead) {
        case 0: wait_vmcnt<0>(); break;
        case 1: wait_vmcnt<(NST > 2 ? 1 : 0) * kStageLoads>(); break;
        default: wait_vmcnt<(NST > 3 ? 2 : 0) * kStageLoads>(); break;
        }
    }

    // One 32-key block: scores, mask, row maximum and rescale, exponentials,
    // then P.V.
    __device__ __forceinline__ static void block(State &st, const _Float16 *kl, const _Float16 *vl, int k0,
                                                 int Lk, int wp0, int qp, float c)
    {
        floatx16 s;
        M::s_product(s, st, kl);
        if (M::needs_mask(k0, Lk, wp0)) M::mask(s, k0, Lk, qp, 4 * ((int)(threadIdx.x & 63) >> 5));
        M::rescale(st, M::block_max(s), c);
        half8 pf[M::kCS];
        float rs[2] = {0.0f, 0.0f};
#pragma unroll
        for (int p = 0; p < M::kPairs; ++p) M::exp_pair(s, pf, rs, p, st.mc, c);
#pragma unroll
        for (int n = 0; n < M::kDBlocks * M::kCS; ++n) {
            const int i = n % M::kDBlocks, cs = n / M::kDBlocks;
            st.oacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(M::vfrag(st, vl, i, cs), pf[cs], st.oacc[i], 0, 0, 0);
        }
        st.l += rs[0] + rs[1];
    }

    __device__ static void run(const SplitArgs &a)
    {
        __shared__ __attribute__((aligned(16))) _Float16 klds[NST][kTile];
        __shared__ __attribute__((aligned(16))) _Float16 vlds[NST][kTile];

        const int lane = threadIdx.x;
        const int col = lane & 31, half = lane >> 5;

        // ---- work item: (b, kv head, split, row block), row block fastest
        const int item = xcd_item(blockIdx.x, a.n_items);
        const int rb = item % a.n_rb;
        int rest = item / a.n_rb;
        const int sp = rest % a.n_splits;
        rest /= a.n_splits;
        const int hk = rest % a.Hkv;
        const int b = rest / a.Hkv;
        const int g = a.groups, Lq = a.Lq, Lk = a.Lk;

        // packed rows of this wavefront; rows past the end are padding (zero
        // queries, never written) and take the last query's position
        const int rows = Lq * g;
        const int R0 = 32 * rb;
        const int R = R0 + col;
        const int qi = R / g;
        const int h = hk * g + (R - qi * g);
        const int R_last = R0 + 31 < rows ? R0 + 31 : rows - 1;
        const int wp0 = R0 / g + a.past_len;       // first query position of the wavefront
        const int wpl = R_last / g + a.past_len;   // last query position of the wavefront
        const int qp = (qi < Lq ? qi : Lq - 1) + a.past_len;

        // keys of this split that the wavefront can see: [ks, ke)
        const int ks = sp * a.split_blocks * kSB;
        int ke = a.kv_vis - ks < a.split_blocks * kSB ? a.kv_vis : ks + a.split_blocks * kSB;
        if (CAUSAL && wpl < ke - 1) ke = wpl + 1;
        const int nb = ke > ks ? (ke - ks + kSB - 1) / kSB : 0;

        const int64_t q_row = (int64_t)a.H * D, kv_row = (int64_t)a.Hkv * D;
        const _Float16 *kbase = a.k + (int64_t)b * Lk * kv_row + (int64_t)hk * D;
        const _Float16 *vbase = a.v + (int64_t)b * Lk * kv_row + (int64_t)hk * D;

        State st;
        M::init(st);
        if (nb > 0) {
            Loads lo;
            init_loads(lo, kv_row);
#pragma unroll
            for (int s = 0; s < NST - 1; ++s)
                if (s < nb) issue_stage(lo, kbase, vbase, kv_row, ks + kSB * s, Lk, klds[s], vlds[s]);
#pragma unroll
            for (int s = 0; s < M::kSteps; ++s) {
                half8 val = {};
                if (qi < Lq)
                    val = *(const half8 *)(a.q + ((int64_t)b * Lq + qi) * q_row + (int64_t)h * D + 16 * s + 8 * half);
                st.qf[s] = val;
            }
            // Q has landed (and with it the first stages): one wait here,
            // rather than a compiler-placed one for Q inside the loop, which
            // would also drain the ring every iteration
            wait_vmcnt<0>();
            M::init_lds_bases(st, (int)threadIdx.x & 63);
            const float c = a.scale_log2;

            int stage = 0;  // ring stage of block t
            for (int t = 0; t < nb; ++t) {
                // refill the stage that block t-1 used, then wait for block t
                const int tn = t + NST - 1;
                if (tn < nb) {
                    const int sn = stage == 0 ? NST - 1 : stage - 1;
                    issue_stage(lo, kbase, vbase, kv_row, ks + kSB * tn, Lk, klds[sn], vlds[sn]);
                }
                wait_stage(nb - 1 - t);
                block(st, klds[stage], vlds[stage], ks + kSB * t, Lk, wp0, qp, c);
                stage = stage == NST - 1 ? 0 : stage + 1;
            }
        }

        // ---- partial result of this split: O_p = acc / l, LSE_p = scale*m + ln l
        // (no visible key: acc = 0, l = 0, m = -inf -> O_p = 0, LSE_p = -inf)
        const float lt = pair_sum(st.l);
        const float inv = 1.0f / (lt > 1e-6f ? lt : 1.0f);
        if (R < rows) {
            const int64_t prow = (((int64_t)b * a.H + h) * Lq + qi) * a.n_splits + sp;
            float *orow = a.ws_o + prow * D;
#pragma unroll
            for (int i = 0; i < M::kDBlocks; ++i)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const float4v out = {st.oacc[i][4 * r4 + 0] * inv, st.oacc[i][4 * r4 + 1] * inv,
                                         st.oacc[i][4 * r4 + 2] * inv, st.oacc[i][4 * r4 + 3] * inv};
                    *(float4v *)(orow + 32 * i + 8 * r4 + 4 * half) = out;
                }
            if (half == 0) a.ws_lse[prow] = st.m * a.scale + __logf(lt);
        }
    }
};

template <int D, bool CAUSAL, int NST>
__global__ __attribute__((amdgpu_flat_work_group_size(64, 64))) void fa_splitkv_kernel(const SplitArgs a)
{
    SplitKernel<D, CAUSAL, NST>::run(a);
}

// Merge of the split partials: M = max_p LSE_p, w_p = exp(LSE_p - M),
// O = sum_p w_p O_p / sum_p w_p, LSE = M + ln sum_p w_p.  A row with no
// visible key anywhere (M = -inf) gets O = 0 and LSE = -inf.
//
// One output row per 16 lanes, 8 consecutive d per lane at D = 128 (4 at
// D = 64), so a 256-thread block merges 16 rows.  The partial LSEs of a row
// are read first, kMergeUnroll at a time with independent loads; then the
// partial outputs, again kMergeUnroll independent loads in flight per lane:
// a merge of few rows is bound by memory latency, not bandwidth.
constexpr int kMergeLanes = 16;   // lanes per output row
constexpr int kMergeRows = 256 / kMergeLanes;
constexpr int kMergeUnroll = 8;

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256))) void fa_splitkv_merge(const MergeArgs a)
{
    constexpr int kPer = D / kMergeLanes;  // d per lane: 8 or 4
    typedef float vec __attribute__((ext_vector_type(kPer)));
    const int64_t row = (int64_t)blockIdx.x * kMergeRows + threadIdx.x / kMergeLanes;
    if (row >= a.n_rows) return;
    const int d0 = kPer * (threadIdx.x % kMergeLanes);
    const int n = a.n_splits;
    const float *lp = a.ws_lse + row * n;
    const float *op = a.ws_o + row * n * D + d0;
    const float ninf = -__builtin_huge_valf();

    float m = ninf;
    for (int p0 = 0; p0 < n; p0 += kMergeUnroll) {
        float v[kMergeUnroll];
#pragma unroll
        for (int j = 0; j < kMergeUnroll; ++j) v[j] = p0 + j < n ? lp[p0 + j] : ninf;
#pragma unroll
        for (int j = 0; j < kMergeUnroll; ++j) m = fmaxf(m, v[j]);
    }
    vec acc = {};
    float wsum = 0.0f;
    if (m != ninf) {
        for (int p0 = 0; p0 < n; p0 += kMergeUnroll) {
            float w[kMergeUnroll];
            vec o[kMergeUnroll];
#pragma unroll
            for (int j = 0; j < kMergeUnroll; ++j) {
                const bool in = p0 + j < n;
                const float l = in ? lp[p0 + j] : ninf;
                // an empty split (LSE_p = -inf) has weight exp(-inf) = 0
                w[j] = expf(l - m);
                o[j] = in ? *(const vec *)(op + (int64_t)(p0 + j) * D) : vec{};
            }
#pragma unroll
            for (int j = 0; j < kMergeUnroll; ++j) {
                wsum += w[j];
                acc += w[j] * o[j];
            }
        }
    }
    const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
    // row = (b*H + h)*Lq + i  ->  O[b][i][h][:]
    const int64_t bh = row / a.Lq, i = row % a.Lq;
    const int64_t b = bh / a.H, h = bh % a.H;
    _Float16 *orow = a.o + ((b * a.Lq + i) * a.H + h) * D + d0;
    const vec r = acc * inv;
#pragma unroll
    for (int j = 0; j < kPer; j += 4) {
        const float4v q4 = {r[j], r[j + 1], r[j + 2], r[j + 3]};
        *(half4 *)(orow + j) = __builtin_convertvector(q4, half4);
    }
    if (a.lse && d0 == 0) a.lse[row] = wsum > 0.0f ? m + logf(wsum) : ninf;
}

constexpr int kStages = 3;  // ring depth of the split kernel

template <int D, bool CAUSAL>
int launch_split(const SplitArgs &s, const MergeArgs &mg, hipStream_t stream)
{
    hipLaunchKernelGGL((fa_splitkv_kernel<D, CAUSAL, kStages>), dim3(s.n_items), dim3(64), 0, stream, s);
    if (hipGetLastError() != hipSuccess) return FA_ERR_LAUNCH;
    const int64_t blocks = (mg.n_rows + kMergeRows - 1) / kMergeRows;
    hipLaunchKernelGGL((fa_splitkv_merge<D>), dim3((unsigned)blocks), dim3(256), 0, stream, mg);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

// Scratch of fa_fwd_splitkv_noalloc: the partial results live in this
// file-scope device array instead of a caller workspace.  Each GPU the
// library runs on holds its own copy for the life of the process.  In host
// code `scratch` names a host-side stand-in, never the device memory: its
// device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and only that address is passed to kernels.
__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxScratchDevices];
std::mutex g_scratch_mutex;
}  // namespace

int splitkv_scratch(void **ptr)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return FA_ERR_DEVICE;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FA_ERR_DEVICE;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return FA_OK;
}

int64_t splitkv_workspace_bytes(int64_t rows_total, int64_t n_splits, int D)
{
    // O_p (fp32, D per row and split) followed by LSE_p (fp32); -1 on overflow
    int64_t cells, o_bytes, lse_bytes, total;
    if (__builtin_mul_overflow(rows_total, n_splits, &cells)) return -1;
    if (__builtin_mul_overflow(cells, (int64_t)D * 4, &o_bytes)) return -1;
    if (__builtin_mul_overflow(cells, (int64_t)4, &lse_bytes)) return -1;
    if (__builtin_add_overflow(o_bytes, lse_bytes, &total)) return -1;
    return total;
}

int launch_splitkv(const Problem &p, int n_splits, void *workspace, hipStream_t stream)
{
    // per-lane tile offsets are 32-bit: 32 K/V rows must span < 2 GiB
    if ((int64_t)p.Hkv * p.D * 2 * kSB > 0x7fffffff) return FA_ERR_SHAPE;
    const int groups = p.H / p.Hkv;
    const int64_t rows = (int64_t)p.Lq * groups;
    const int64_t n_rb = (rows + 31) / 32;
    const int64_t items = (int64_t)p.B * p.Hkv * n_rb * n_splits;
    if (rows > 0x7fffffff - 64 || items > 0x7fffffff) return FA_ERR_SHAPE;
    const int64_t n_rows = (int64_t)p.B * p.H * p.Lq;
    if ((n_rows + kMergeRows - 1) / kMergeRows > 0x7fffffff) return FA_ERR_SHAPE;

    // visible keys: all of them, or (causal) up to the last query's position
    int64_t kv_vis = p.Lk;
    if (p.causal) {
        const int64_t last = (int64_t)p.Lq + p.past_len;
        kv_vis = last < 0 ? 0 : (last < p.Lk ? last : p.Lk);
    }
    const int64_t blocks = (kv_vis + kSB - 1) / kSB;
    const int64_t split_blocks = (blocks + n_splits - 1) / n_splits;

    SplitArgs s;
    s.q = (const _Float16 *)p.q;
    s.k = (const _Float16 *)p.k;
    s.v = (const _Float16 *)p.v;
    s.ws_o = (float *)workspace;
    s.ws_lse = (float *)((char *)workspace + n_rows * n_splits * p.D * 4);
    s.Lq = p.Lq;
    s.Lk = p.Lk;
    s.past_len = p.past_len;
    s.H = p.H;
    s.Hkv = p.Hkv;
    s.groups = groups;
    s.n_rb = (int)n_rb;
    s.n_splits = n_splits;
    s.n_items = (int)items;
    s.split_blocks = (int)split_blocks;
    s.kv_vis = (int)kv_vis;
    s.scale = p.scale;
    s.scale_log2 = p.scale * 1.4426950408889634f;

    MergeArgs mg;
    mg.ws_o = s.ws_o;
    mg.ws_lse = s.ws_lse;
    mg.o = (_Float16 *)p.o;
    mg.lse = p.lse;
    mg.Lq = p.Lq;
    mg.H = p.H;
    mg.n_splits = n_splits;
    mg.n_rows = n_rows;

    if (p.D == 64) return p.causal ? launch_split<64, true>(s, mg, stream) : launch_split<64, false>(s, mg, stream);
    return p.causal ? launch_split<128, true>(s, mg, stream) : launch_split<128, false>(s, mg, stream);
}

}  // namespace fa
