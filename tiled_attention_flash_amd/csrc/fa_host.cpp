// fa_host.cpp -- the C-ABI front end of libfa.so: argument validation and
// dispatch.  Every check runs before any HIP call, so a rejected call never
// touches the device (and the checks can be exercised on a host without one).
#include <math.h>
#include <stdint.h>

#include "fa.h"
#include "fa_internal.h"

namespace {

bool mul_overflows(int64_t a, int64_t b, int64_t *out) { return __builtin_mul_overflow(a, b, out); }

// Element count of a 4-D tensor, or -1 on int64 overflow.
int64_t elems4(int a, int b, int c, int d)
{
    int64_t x;
    if (mul_overflows(a, b, &x) || mul_overflows(x, c, &x) || mul_overflows(x, d, &x)) return -1;
    return x;
}

bool overlaps(const void *a, int64_t a_bytes, const void *b, int64_t b_bytes)
{
    if (!a || !b || a_bytes <= 0 || b_bytes <= 0) return false;
    uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + (uintptr_t)b_bytes && b0 < a0 + (uintptr_t)a_bytes;
}

bool misaligned(const void *p, uintptr_t to) { return ((uintptr_t)p & (to - 1)) != 0; }

// Shared argument validation of every forward entry point.  in_size is the
// byte size of a q/k/v element (2 for fp16, 1 for E4M3); o is always fp16.
// Returns FA_OK with *p filled in, FA_OK with *empty set when there is
// nothing to compute, or an error status.
int validate(const void *q, const void *k, const void *v, void *o, float *lse, int B, int Lq, int Lk,
             int H, int Hkv, int D, int causal, int past_len, float scale, fa::Problem *p, bool *empty,
             int in_size = 2)
{
    *empty = false;
    if (B < 0 || Lq < 0 || Lk < 0 || H < 0 || Hkv < 0 || D < 0) return FA_ERR_SHAPE;
    if (H <= 0 || Hkv <= 0 || H % Hkv != 0) return FA_ERR_GQA;
    if (D != 64 && D != 128) return FA_ERR_HEADDIM;
    if (!isfinite(scale) || !(scale > 0.0f)) return FA_ERR_SCALE;
    // positions i + past_len and key indices stay far from int overflow
    if (Lq > (1 << 30) || Lk > (1 << 30) || past_len > (1 << 30) || past_len < -(1 << 30))
        return FA_ERR_SHAPE;

    int64_t q_elems = elems4(B, Lq, H, D);
    int64_t kv_elems = elems4(B, Lk, Hkv, D);
    int64_t lse_elems = elems4(B, H, Lq, 1);
    if (q_elems < 0 || kv_elems < 0 || lse_elems < 0 || q_elems > INT64_MAX / 4 ||
        kv_elems > INT64_MAX / 4)
        return FA_ERR_SHAPE;
    if (B == 0 || Lq == 0) {  // nothing to compute; pointers may be null
        *empty = true;
        return FA_OK;
    }

    if (!q || !o || (Lk > 0 && (!k || !v))) return FA_ERR_NULLPTR;
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(o, 16) ||
        misaligned(lse, 4))
        return FA_ERR_ALIGN;

    const int64_t q_bytes = q_elems * in_size, kv_bytes = kv_elems * in_size;
    const int64_t o_bytes = q_elems * 2, lse_bytes = lse_elems * 4;
    if (overlaps(o, o_bytes, q, q_bytes) || overlaps(o, o_bytes, k, kv_bytes) ||
        overlaps(o, o_bytes, v, kv_bytes) || overlaps(o, o_bytes, lse, lse_bytes) ||
        overlaps(lse, lse_bytes, q, q_bytes) || overlaps(lse, lse_bytes, k, kv_bytes) ||
        overlaps(lse, lse_bytes, v, kv_bytes))
        return FA_ERR_ALIAS;

    *p = fa::Problem{q, k, v, o, lse, B, Lq, Lk, H, Hkv, D, causal != 0, causal ? past_len : 0, scale};
    return FA_OK;
}

int forward(const void *q, const void *k, const void *v, void *o, float *lse, int B, int Lq, int Lk,
            int H, int Hkv, int D, int causal, int past_len, float scale, hipStream_t stream)
{
    fa::Problem p;
    bool empty;
    const int st = validate(q, k, v, o, lse, B, Lq, Lk, H, Hkv, D, causal, past_len, scale, &p, &empty);
    if (st != FA_OK || empty) return st;
    return fa::launch_forward(p, stream);
}

// Keys that some query row can see: all Lk, or (causal) up to the last
// query's position Lq - 1 + past_len.
int64_t visible_keys(int Lq, int Lk, int causal, int past_len)
{
    if (!causal) return Lk;
    const int64_t last = (int64_t)Lq + past_len;  // one past the last visible key
    return last < 0 ? 0 : (last < Lk ? last : Lk);
}

constexpr int kMaxSplits = 4096;

// The library's choice of key splits.  Each (b, kv head, row block, split)
// work item is one wavefront holding a 3-stage ring of 32-key K and V tiles
// in LDS (384*D bytes), so 160 KiB of LDS keeps `slots` of them resident on
// the 256 compute units.  Work items run in rounds of `slots`; a round costs
// about the split's length in 32-key blocks plus two blocks of fixed work,
// and a last round that is only partly full costs as much as a full one.
// The choice minimises rounds * (blocks per split + 2) over 1..64 splits
// (the merge reads every split's partial result), with no split shorter
// than four blocks; ties go to fewer splits.
int default_splits(int B, int Lq, int Lk, int H, int Hkv, int D, int causal, int past_len)
{
    if (B <= 0 || Lq <= 0 || H <= 0 || Hkv <= 0 || H % Hkv != 0 || (D != 64 && D != 128)) return 1;
    const int64_t rows = (int64_t)Lq * (H / Hkv);
    const int64_t base = (int64_t)B * Hkv * ((rows + 31) / 32);
    const int64_t blocks = (visible_keys(Lq, Lk, causal, past_len) + 31) / 32;
    const int64_t slots = 256 * ((160 * 1024) / (384 * D));
    int64_t cap = blocks / 4;
    if (cap > 64) cap = 64;
    if (cap < 1) cap = 1;
    int best = 1;
    int64_t best_cost = -1;
    for (int64_t n = 1; n <= cap; ++n) {
        const int64_t rounds = (base * n + slots - 1) / slots;
        const int64_t cost = rounds * ((blocks + n - 1) / n + 2);
        if (best_cost < 0 || cost < best_cost) {
            best_cost = cost;
            best = (int)n;
        }
    }
    return best;
}

}  // namespace

extern "C" int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                      int L, int H, int Hkv, int D, int causal, float scale, hipStream_t stream)
{
    return forward(q, k, v, o, lse, B, L, L, H, Hkv, D, causal, 0, scale, stream);
}

extern "C" int fa_fwd_kv(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                         int Lq, int Lk, int H, int Hkv, int D, int causal, int past_len,
                         float scale, hipStream_t stream)
{
    return forward(q, k, v, o, lse, B, Lq, Lk, H, Hkv, D, causal, past_len, scale, stream);
}

extern "C" int fa_fwd_fp8(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                          int Lq, int Lk, int H, int Hkv, int D, int causal, int past_len,
                          float scale, float q_descale, float k_descale, float v_descale,
                          hipStream_t stream)
{
    fa::Problem p;
    bool empty;
    const int st =
        validate(q, k, v, o, lse, B, Lq, Lk, H, Hkv, D, causal, past_len, scale, &p, &empty, 1);
    if (st != FA_OK) return st;
    for (float d : {q_descale, k_descale, v_descale})
        if (!isfinite(d) || !(d > 0.0f)) return FA_ERR_SCALE;
    if (!isfinite(scale * q_descale * k_descale) || !(scale * q_descale * k_descale > 0.0f))
        return FA_ERR_SCALE;
    if (empty) return FA_OK;
    return fa::launch_forward_fp8(p, fa::Fp8Descale{q_descale, k_descale, v_descale}, stream);
}

extern "C" int fa_splitkv_splits(int B, int Lq, int Lk, int H, int Hkv, int D, int causal,
                                 int past_len)
{
    return default_splits(B, Lq, Lk, H, Hkv, D, causal, past_len);
}

extern "C" long long fa_splitkv_workspace_bytes(int B, int Lq, int H, int D, int n_splits)
{
    if (B < 0 || Lq < 0 || H < 0 || (D != 64 && D != 128) || n_splits < 1 || n_splits > kMaxSplits)
        return -1;
    const int64_t rows = elems4(B, H, Lq, 1);
    if (rows < 0) return -1;
    return (long long)fa::splitkv_workspace_bytes(rows, n_splits, D);
}

extern "C" int fa_fwd_splitkv(const void *q, const void *k, const void *v, void *o, float *lse,
                              int B, int Lq, int Lk, int H, int Hkv, int D, int causal,
                              int past_len, float scale, int n_splits, void *workspace,
                              long long workspace_bytes, hipStream_t stream)
{
    fa::Problem p;
    bool empty;
    const int st = validate(q, k, v, o, lse, B, Lq, Lk, H, Hkv, D, causal, past_len, scale, &p, &empty);
    if (st != FA_OK) return st;
    if (n_splits < 0 || n_splits > kMaxSplits) return FA_ERR_SHAPE;
    if (empty) return FA_OK;
    if (n_splits == 0) n_splits = default_splits(B, Lq, Lk, H, Hkv, D, causal, past_len);
    const int64_t need = fa::splitkv_workspace_bytes(elems4(B, H, Lq, 1), n_splits, D);
    if (need < 0) return FA_ERR_SHAPE;
    if (!workspace || workspace_bytes < need || misaligned(workspace, 16)) return FA_ERR_WORKSPACE;
    const int64_t q_bytes = elems4(B, Lq, H, D) * 2, kv_bytes = elems4(B, Lk, Hkv, D) * 2;
    const int64_t lse_bytes = elems4(B, H, Lq, 1) * 4;
    if (overlaps(workspace, need, q, q_bytes) || overlaps(workspace, need, k, kv_bytes) ||
        overlaps(workspace, need, v, kv_bytes) || overlaps(workspace, need, o, q_bytes) ||
        overlaps(workspace, need, lse, lse_bytes))
        return FA_ERR_ALIAS;
    return fa::launch_splitkv(p, n_splits, workspace, stream);
}

extern "C" int fa_fwd_splitkv_noalloc(const void *q, const void *k, const void *v, void *o,
                                      float *lse, int B, int Lq, int Lk, int H, int Hkv, int D,
                                      int causal, int past_len, float scale, int n_splits,
                                      hipStream_t stream)
{
    fa::Problem p;
    bool empty;
    const int st = validate(q, k, v, o, lse, B, Lq, Lk, H, Hkv, D, causal, past_len, scale, &p, &empty);
    if (st != FA_OK) return st;
    if (n_splits < 0 || n_splits > kMaxSplits) return FA_ERR_SHAPE;
    if (empty) return FA_OK;
    if (n_splits == 0) n_splits = default_splits(B, Lq, Lk, H, Hkv, D, causal, past_len);
    const int64_t need = fa::splitkv_workspace_bytes(elems4(B, H, Lq, 1), n_splits, D);
    if (need < 0) return FA_ERR_SHAPE;
    if (need > fa::kScratchBytes) return FA_ERR_SCRATCH;  // checked before any HIP call
    void *scratch = nullptr;
    const int sst = fa::splitkv_scratch(&scratch);
    if (sst != FA_OK) return sst;
    return fa::launch_splitkv(p, n_splits, scratch, stream);
}

namespace {

// Validation and dispatch of the backward entry points.  Every pointer a
// nonempty problem reads or writes must be non-NULL: q, o, dout, lse, delta
// and dq when there are query rows, k, v, dk and dv when there are keys.
int backward(const void *q, const void *k, const void *v, const void *o, const void *dout,
             const float *lse, float *delta, void *dq, void *dk, void *dv, int B, int Lq, int Lk,
             int H, int Hkv, int D, int causal, int past_len, float scale, hipStream_t stream)
{
    if (B < 0 || Lq < 0 || Lk < 0 || H < 0 || Hkv < 0 || D < 0) return FA_ERR_SHAPE;
    if (H <= 0 || Hkv <= 0 || H % Hkv != 0) return FA_ERR_GQA;
    if (D != 64 && D != 128) return FA_ERR_HEADDIM;
    if (!isfinite(scale) || !(scale > 0.0f)) return FA_ERR_SCALE;
    // positions i + past_len and key indices stay far from int overflow
    if (Lq > (1 << 30) || Lk > (1 << 30) || past_len > (1 << 30) || past_len < -(1 << 30))
        return FA_ERR_SHAPE;
    const int64_t q_elems = elems4(B, Lq, H, D), kv_elems = elems4(B, Lk, Hkv, D);
    const int64_t row_elems = elems4(B, H, Lq, 1);
    if (q_elems < 0 || kv_elems < 0 || row_elems < 0 || q_elems > INT64_MAX / 4 ||
        kv_elems > INT64_MAX / 4)
        return FA_ERR_SHAPE;
    if (B == 0 || (Lq == 0 && Lk == 0)) return FA_OK;

    if (Lq > 0 && (!q || !o || !dout || !lse || !delta || !dq)) return FA_ERR_NULLPTR;
    if (Lk > 0 && (!k || !v || !dk || !dv)) return FA_ERR_NULLPTR;
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(o, 16) ||
        misaligned(dout, 16) || misaligned(dq, 16) || misaligned(dk, 16) || misaligned(dv, 16) ||
        misaligned(lse, 4) || misaligned(delta, 4))
        return FA_ERR_ALIGN;

    // every written buffer is disjoint from every other buffer
    const int64_t qb = q_elems * 2, kvb = kv_elems * 2, rb = row_elems * 4;
    const void *in[6] = {q, k, v, o, dout, lse};
    const int64_t in_bytes[6] = {qb, kvb, kvb, qb, qb, rb};
    void *out[4] = {delta, dq, dk, dv};
    const int64_t out_bytes[4] = {rb, qb, kvb, kvb};
    for (int i = 0; i < 4; ++i) {
        for (int j = 0; j < 6; ++j)
            if (overlaps(out[i], out_bytes[i], in[j], in_bytes[j])) return FA_ERR_ALIAS;
        for (int j = i + 1; j < 4; ++j)
            if (overlaps(out[i], out_bytes[i], out[j], out_bytes[j])) return FA_ERR_ALIAS;
    }
    fa::BwdProblem p{q, k, v, o, dout, lse, delta, dq, dk, dv, B, Lq, Lk, H, Hkv, D, causal != 0,
                     causal ? past_len : 0, scale};
    return fa::launch_backward(p, stream);
}

}  // namespace

extern "C" int fa_bwd(const void *q, const void *k, const void *v, const void *o,
                      const void *dout, const float *lse, float *delta, void *dq, void *dk,
                      void *dv, int B, int L, int H, int Hkv, int D, int causal, float scale,
                      hipStream_t stream)
{
    return backward(q, k, v, o, dout, lse, delta, dq, dk, dv, B, L, L, H, Hkv, D, causal, 0, scale,
                    stream);
}

extern "C" int fa_bwd_kv(const void *q, const void *k, const void *v, const void *o,
                         const void *dout, const float *lse, float *delta, void *dq, void *dk,
                         void *dv, int B, int Lq, int Lk, int H, int Hkv, int D, int causal,
                         int past_len, float scale, hipStream_t stream)
{
    return backward(q, k, v, o, dout, lse, delta, dq, dk, dv, B, Lq, Lk, H, Hkv, D, causal, past_len,
                    scale, stream);
}

extern "C" const char *fa_status_string(int status)
{
    switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULLPTR: return "FA_ERR_NULLPTR: q, k, v or o is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: negative size, size overflow, or |past_len| > 2^30";
    case FA_ERR_GQA: return "FA_ERR_GQA: H and Hkv must be positive and H a multiple of Hkv";
    case FA_ERR_HEADDIM: return "FA_ERR_HEADDIM: head dimension must be 64 or 128";
    case FA_ERR_SCALE: return "FA_ERR_SCALE: scale (and fp8 descales) must be finite and > 0";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: q/k/v/o need 16-byte, lse 4-byte alignment";
    case FA_ERR_ALIAS: return "FA_ERR_ALIAS: o or lse overlaps another tensor";
    case FA_ERR_LAUNCH: return "FA_ERR_LAUNCH: the HIP runtime rejected the kernel launch";
    case FA_ERR_DEVICE: return "FA_ERR_DEVICE: could not query the current device";
    case FA_ERR_WORKSPACE:
        return "FA_ERR_WORKSPACE: workspace is NULL, smaller than fa_splitkv_workspace_bytes, "
               "or not 16-byte aligned";
    case FA_ERR_SCRATCH:
        return "FA_ERR_SCRATCH: fa_fwd_splitkv_noalloc needs more than its static scratch "
               "(FA_SPLITKV_SCRATCH_BYTES = 16 MiB) holds; use fa_fwd_splitkv with a workspace "
               "or fewer splits";
    default: return "FA_ERR_UNKNOWN";
    }
}

extern "C" int fa_abi_version(void) { return 7; }
