/*
 * fa.h -- C ABI of libfa.so, the attention forward pass (fp16 and fp8
 * inputs, split-KV decoding) and its backward pass for AMD Instinct MI355X
 * (gfx950).
 *
 * Operation (page "使用 TileLang 在 AMD GPU 上快速开发高性能 Flash Attention",
 * sections "核心公式与计算流程" and "K/V Tile 遍历与核心计算"):
 *
 *   for every batch b, query head h and query row i:
 *     hk    = h / (H / Hkv)                         grouped-query K/V head
 *     s_j   = scale * sum_d Q[b,i,h,d] * K[b,j,hk,d]  for visible keys j
 *             (all j < L; with causal != 0 only j <= i)
 *     O[b,i,h,:] = sum_j softmax_j(s) * V[b,j,hk,:]
 *     LSE[b,h,i] = ln( sum_j exp(s_j) )             natural log, scaled scores
 *
 * computed tile by tile with an fp32 online softmax (running row maximum,
 * running row sum, rescaled fp32 output accumulator), fp16 inputs, fp16
 * probabilities into the second product, fp32 accumulation, and the output
 * rounded to fp16 with round-to-nearest-even.
 *
 * The library allocates nothing, keeps no per-call state and never
 * synchronises the device: every call only validates its arguments and
 * enqueues kernels on `stream`.  It is reentrant and thread-safe.
 */
#ifndef FA_H
#define FA_H

#ifdef __cplusplus
extern "C" {
#endif

#ifndef FA_API
#define FA_API __attribute__((visibility("default")))
#endif

/* Same definition as the HIP runtime's own handle type, so this header does
 * not need the HIP headers. 0 (NULL) is the null stream. */
typedef struct ihipStream_t *hipStream_t;

enum fa_status {
    FA_OK = 0,
    FA_ERR_NULLPTR = 1,  /* q, k, v or o is NULL                                  */
    FA_ERR_SHAPE = 2,    /* a size is negative or overflows int64; fa_fwd_kv also:
                            Lq or Lk > 2^30, or |past_len| > 2^30; the forward
                            entry points: 64 rows of K span 2 GiB or more;
                            fa_bwd: 256 rows of Q do (H*D >= 2^22)          */
    FA_ERR_GQA = 3,      /* Hkv <= 0, H <= 0, or H not a multiple of Hkv           */
    FA_ERR_HEADDIM = 4,  /* D is not 64 or 128                                     */
    FA_ERR_SCALE = 5,    /* scale is not finite or not > 0                         */
    FA_ERR_ALIGN = 6,    /* a tensor pointer is not 16-byte aligned (lse: 4-byte)  */
    FA_ERR_ALIAS = 7,    /* the byte range of o or lse overlaps q, k, v or each other */
    FA_ERR_LAUNCH = 8,   /* the HIP runtime rejected the launch                    */
    FA_ERR_DEVICE = 9,   /* the current device could not be queried                */
    FA_ERR_WORKSPACE = 10, /* fa_fwd_splitkv: workspace NULL, too small or not
                             16-byte aligned                                       */
    FA_ERR_SCRATCH = 11   /* fa_fwd_splitkv_noalloc: the partial results need more
                             than FA_SPLITKV_SCRATCH_BYTES                         */
};

/* Size of the static device scratch of fa_fwd_splitkv_noalloc (16 MiB). */
#define FA_SPLITKV_SCRATCH_BYTES (16LL << 20)

/*
 * fa_fwd -- attention forward pass.
 *
 * q    device pointer, fp16 (IEEE binary16), contiguous [B][L][H][D]   (read)
 * k    device pointer, fp16, contiguous [B][L][Hkv][D]                 (read)
 * v    device pointer, fp16, contiguous [B][L][Hkv][D]                 (read)
 * o    device pointer, fp16, contiguous [B][L][H][D]                   (written)
 * lse  device pointer, fp32, contiguous [B][H][L], or NULL to skip it  (written)
 *      LSE[b,h,i] = ln sum_{visible j} exp(s_ij), with s_ij the scaled score.
 * B, L, H, Hkv, D   batch, sequence length (queries = keys), query heads,
 *      K/V heads (H % Hkv == 0; query head h uses K/V head h / (H/Hkv)),
 *      head dimension (64 or 128).
 * causal  nonzero: key j is visible to query i iff j <= i (top-left aligned,
 *      which is also bottom-right aligned because queries and keys have the
 *      same length).
 * scale   multiplier of Q.K; must be finite and > 0 (1/sqrt(D) is the usual).
 * stream  HIP stream the kernels are enqueued on.
 *
 * Ownership: the caller allocates and frees every buffer; they must stay
 * valid until the enqueued work has completed.  o and lse must not overlap
 * q, k, v or each other (checked on the pointers' byte ranges).
 *
 * Returns FA_OK once the work is enqueued, or an fa_status error, in which
 * case nothing was launched and no buffer was touched.  All argument checks
 * happen before any HIP call.  With causal != 0 the grid is sized to the
 * workgroups the current device holds at once (its compute units, queried
 * once per device); FA_ERR_DEVICE if the runtime cannot report them.  B == 0 or L == 0 returns FA_OK and launches
 * nothing.  Faults inside the kernel surface at the caller's next
 * synchronisation on `stream`.
 */
FA_API int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
           int B, int L, int H, int Hkv, int D, int causal, float scale,
           hipStream_t stream);

/*
 * fa_fwd_kv -- attention forward pass with Lq query rows and Lk key rows, for
 * queries that follow past_len earlier positions of the key sequence (a
 * prefill after a cached prefix: past_len = Lk - Lq).
 *
 * Mask (page "TileLang性能分析报告：H100上FlashAttention吞吐量达1.2PFlops",
 * section "因果掩码优化"): query row i sits at position i + past_len, and with
 * causal != 0 it sees key j iff j <= i + past_len.  Without the mask every
 * query sees all Lk keys and past_len is ignored.  A row that sees no key
 * (i + past_len < 0, or Lk == 0) gets O = 0 -- the division guard of the
 * output stage applied to an empty sum -- and LSE = -inf.
 *
 * q    device pointer, fp16, contiguous [B][Lq][H][D]                  (read)
 * k    device pointer, fp16, contiguous [B][Lk][Hkv][D]                (read)
 * v    device pointer, fp16, contiguous [B][Lk][Hkv][D]                (read)
 *      k and v may be NULL when Lk == 0.
 * o    device pointer, fp16, contiguous [B][Lq][H][D]                  (written)
 * lse  device pointer, fp32, contiguous [B][H][Lq], or NULL            (written)
 * B, Lq, Lk, H, Hkv, D   as for fa_fwd, with Lq, Lk <= 2^30.
 * causal, past_len       see above; |past_len| <= 2^30.
 * scale, stream          as for fa_fwd.
 *
 * Ownership, aliasing and error behaviour are those of fa_fwd;
 * fa_fwd(..., L, ...) is fa_fwd_kv(..., L, L, ..., past_len = 0, ...).
 * B == 0 or Lq == 0 returns FA_OK and launches nothing.
 */
FA_API int fa_fwd_kv(const void *q, const void *k, const void *v, void *o, float *lse,
              int B, int Lq, int Lk, int H, int Hkv, int D, int causal, int past_len,
              float scale, hipStream_t stream);

/*
 * fa_fwd_fp8 -- the operation of fa_fwd_kv on 8-bit floating-point inputs
 * (page "TileLang性能分析报告：H100上FlashAttention吞吐量达1.2PFlops", section
 * "生产环境部署建议", names FP8 mixed precision as the next step for
 * throughput).  q, k and v hold OCP FP8 E4M3 codes ("e4m3fn": 1 sign bit,
 * 4 exponent bits with bias 7, 3 fraction bits, no infinities, S.1111.111 is
 * NaN, largest finite 448), one descale factor per tensor: the value of a
 * code c of q is q_descale * e4m3(c), likewise for k and v.  The scores are
 * s_j = scale * q_descale * k_descale * sum_d q[i,d] * k[j,d] (exact E4M3
 * products, fp32 accumulation), and
 *   O   = v_descale * sum_j softmax_j(s) * v[j,:],   LSE = ln sum_j exp(s_j).
 *
 * The probabilities enter the second product as E4M3 (each stored as 8 times
 * its weight relative to the row's running maximum: relative rounding error
 * at most 2^-4 for weights down to 2^-9 of the maximum's); the row sums and
 * the LSE use the unrounded fp32 probabilities.  O is fp16 (round to nearest
 * even), LSE fp32, as for fa_fwd_kv.
 *
 * q       device pointer, E4M3 bytes, contiguous [B][Lq][H][D]      (read)
 * k, v    device pointers, E4M3 bytes, contiguous [B][Lk][Hkv][D]   (read)
 *         (NULL allowed when Lk == 0)
 * o       device pointer, fp16, contiguous [B][Lq][H][D]            (written)
 * lse     device pointer, fp32, contiguous [B][H][Lq], or NULL      (written)
 * B .. scale, stream       as for fa_fwd_kv.
 * q_descale, k_descale, v_descale   finite and > 0 (and scale * q_descale *
 *         k_descale finite and > 0), else FA_ERR_SCALE.
 *
 * Ownership, alignment (16 bytes for q, k, v, o; 4 for lse), aliasing and
 * the other errors as for fa_fwd_kv; the byte ranges of q, k, v are one byte
 * per element.  B == 0 or Lq == 0 returns FA_OK and launches nothing.
 */
FA_API int fa_fwd_fp8(const void *q, const void *k, const void *v, void *o, float *lse,
                      int B, int Lq, int Lk, int H, int Hkv, int D, int causal, int past_len,
                      float scale, float q_descale, float k_descale, float v_descale,
                      hipStream_t stream);

/*
 * fa_fwd_splitkv -- the same operation as fa_fwd_kv, computed by splitting
 * the key sequence (flash decoding; page "TileLang性能分析报告：H100上
 * FlashAttention吞吐量达1.2PFlops", section "生产环境部署建议", which names it
 * for inference).  Meant for few query rows against many keys (decoding one
 * or a few tokens after a long cache), where the forward kernel's work items
 * -- one per block of query rows -- are too few to fill the GPU.
 *
 * Each of n_splits contiguous ranges of the visible keys is processed by
 * separate wavefronts, which write a partial result per query row and split
 * p: LSE_p = ln sum_{j in p} exp(s_j) and O_p = sum_{j in p} exp(s_j - LSE_p)
 * V_j (fp32).  A second kernel merges them exactly:
 *   LSE = ln sum_p exp(LSE_p),   O = sum_p exp(LSE_p - LSE) O_p,
 * taking the largest LSE_p out first.  The per-split arithmetic (fp16
 * products with fp32 accumulation, fp32 online softmax, fp16 probabilities
 * into the second product) is that of fa_fwd; only the summation order over
 * keys differs.  Mask, past_len, empty rows (O = 0, LSE = -inf) and the
 * output rounding are as for fa_fwd_kv.
 *
 * Arguments q .. stream as for fa_fwd_kv, plus:
 * n_splits   number of key splits, 1..4096; 0 = the library's choice,
 *            fa_splitkv_splits(...).  Splits left empty by the mask or by
 *            rounding contribute nothing.
 * workspace  device pointer, 16-byte aligned, at least
 *            fa_splitkv_workspace_bytes(B, Lq, H, D, n_splits) bytes (with
 *            n_splits after the substitution of 0), owned by the caller,
 *            overwritten by the call; it must not overlap any other buffer.
 *            Calls that share a workspace must be ordered on one stream.
 * workspace_bytes  its size.
 *
 * Errors: those of fa_fwd_kv; FA_ERR_SHAPE for n_splits outside 0..4096;
 * FA_ERR_WORKSPACE for a NULL, short or misaligned workspace; FA_ERR_ALIAS
 * when it overlaps another buffer.  B == 0 or Lq == 0 returns FA_OK and
 * launches nothing (the workspace may then be NULL).
 */
FA_API int fa_fwd_splitkv(const void *q, const void *k, const void *v, void *o, float *lse,
                          int B, int Lq, int Lk, int H, int Hkv, int D, int causal, int past_len,
                          float scale, int n_splits, void *workspace, long long workspace_bytes,
                          hipStream_t stream);

/*
 * fa_fwd_splitkv_noalloc -- fa_fwd_splitkv without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  It allocates
 * nothing: the partial results go to a static device array of
 * FA_SPLITKV_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends.  Same kernels, same results (bitwise) as
 * fa_fwd_splitkv with the same n_splits.
 *
 * Arguments and errors as for fa_fwd_splitkv, without workspace and
 * workspace_bytes; in addition FA_ERR_SCRATCH (checked before any HIP call)
 * when fa_splitkv_workspace_bytes(B, Lq, H, D, n_splits) exceeds
 * FA_SPLITKV_SCRATCH_BYTES -- pass fewer splits, or use fa_fwd_splitkv --
 * and FA_ERR_DEVICE if the scratch's device address cannot be obtained.
 *
 * Every call on one GPU uses that GPU's one scratch array: calls that may
 * run concurrently on one GPU (on different streams, or from several host
 * threads without ordering) race on it and must not overlap.  Calls ordered
 * on one stream are safe.  Nothing in the scratch needs to start at zero;
 * each call overwrites what it reads.
 */
FA_API int fa_fwd_splitkv_noalloc(const void *q, const void *k, const void *v, void *o,
                                  float *lse, int B, int Lq, int Lk, int H, int Hkv, int D,
                                  int causal, int past_len, float scale, int n_splits,
                                  hipStream_t stream);

/* The number of key splits fa_fwd_splitkv uses when passed n_splits = 0.
 * Work items (one wavefront per row block and split) run in rounds of as
 * many as the GPU holds at once (256 compute units x 160 KiB of LDS over
 * 384*D bytes per wavefront); the choice minimises rounds x (32-key blocks
 * per split + 2) over 1..64 splits, no split shorter than four blocks, ties
 * to fewer splits.  At least 1.  Pure host arithmetic; never fails. */
FA_API int fa_splitkv_splits(int B, int Lq, int Lk, int H, int Hkv, int D, int causal,
                             int past_len);

/* Workspace bytes fa_fwd_splitkv needs: B*H*Lq*n_splits*(D + 1)*4 (fp32
 * partial outputs [B][H][Lq][n_splits][D], then partial LSEs
 * [B][H][Lq][n_splits]).  -1 for invalid arguments (a negative size, D not
 * 64 or 128, n_splits outside 1..4096) or int64 overflow. */
FA_API long long fa_splitkv_workspace_bytes(int B, int Lq, int H, int D, int n_splits);

/*
 * fa_bwd -- attention backward pass: the gradients of sum(O * dout) with
 * respect to q, k and v, for queries and keys of equal length L (page
 * "TileLang 与机器学习训练：反向传播算子优化案例", section "算子拆分与流水线设计":
 * a preprocess computing Delta from O and dO, then the gradient kernels,
 * which consume lse and Delta).  Per row i of query head h (K/V head hk):
 *   P_ij    = exp(s_ij - LSE[b,h,i])        s_ij as in fa_fwd, masked keys 0
 *   Delta_i = sum_d O[b,i,h,d] * dout[b,i,h,d]
 *   dS_ij   = P_ij * (sum_d dout[b,i,h,d] * V[b,j,hk,d] - Delta_i)
 *   dq[b,i,h,:]  = scale * sum_j dS_ij * K[b,j,hk,:]
 *   dk[b,j,hk,:] = scale * sum over (i, h in hk's group) of dS_ij * Q[b,i,h,:]
 *   dv[b,j,hk,:] = sum over (i, h in hk's group) of P_ij * dout[b,i,h,:]
 * computed with fp16 MFMA operands (P and dS rounded to fp16) and fp32
 * accumulation; the gradients are written as fp16 (round to nearest even).
 *
 * q, k, v     device pointers, the forward's inputs (layouts as for fa_fwd)
 * o           device pointer, fp16 [B][L][H][D]: the forward's output   (read)
 * dout        device pointer, fp16 [B][L][H][D]: gradient of the output (read)
 * lse         device pointer, fp32 [B][H][L]: the forward's LSE         (read)
 * delta       device pointer, fp32 [B][H][L]: receives Delta        (written)
 * dq          device pointer, fp16 [B][L][H][D]                     (written)
 * dk, dv      device pointers, fp16 [B][L][Hkv][D]                  (written)
 * B, L, H, Hkv, D, causal, scale, stream   as for fa_fwd.
 *
 * Ownership, sizes and errors as for fa_fwd; every pointer must be non-NULL
 * (FA_ERR_NULLPTR), 16-byte aligned (lse and delta: 4-byte; FA_ERR_ALIGN),
 * and the written buffers (delta, dq, dk, dv) must not overlap any other
 * buffer (FA_ERR_ALIAS).  B == 0 or L == 0 returns FA_OK and launches
 * nothing.  No atomics: results are deterministic.
 */
FA_API int fa_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
                  const float *lse, float *delta, void *dq, void *dk, void *dv, int B, int L,
                  int H, int Hkv, int D, int causal, float scale, hipStream_t stream);

/*
 * fa_bwd_kv -- the backward pass of fa_fwd_kv: queries and keys of
 * different lengths (cross-attention; queries that follow past_len cached
 * positions).  The same computation as fa_bwd, with query row i at position
 * i + past_len among the keys: under the causal mask it keeps key j iff
 * i + past_len >= j (past_len is ignored without the mask), exactly as in
 * fa_fwd_kv.  A row that keeps no key has dq = 0 and adds nothing to dk and
 * dv; a key that no row keeps gets dk = dv = 0.
 *
 * q, o, dout, dq   device pointers, fp16 [B][Lq][H][D]
 * k, v, dk, dv     device pointers, fp16 [B][Lk][Hkv][D]
 * lse, delta       device pointers, fp32 [B][H][Lq]
 * B, Lq, Lk, H, Hkv, D, causal, past_len, scale, stream   as for fa_fwd_kv.
 *
 * Ownership and errors as for fa_bwd; the pointers a problem touches must be
 * non-NULL (q, o, dout, lse, delta, dq when Lq > 0; k, v, dk, dv when
 * Lk > 0).  B == 0, or Lq == Lk == 0, returns FA_OK and launches nothing;
 * Lq == 0 with keys writes dk = dv = 0.  fa_bwd(..., L, ...) is
 * fa_bwd_kv(..., L, L, ..., past_len = 0, ...).
 */
FA_API int fa_bwd_kv(const void *q, const void *k, const void *v, const void *o, const void *dout,
                     const float *lse, float *delta, void *dq, void *dk, void *dv, int B, int Lq,
                     int Lk, int H, int Hkv, int D, int causal, int past_len, float scale,
                     hipStream_t stream);

/* Human-readable name of an fa_status value (static storage, never NULL). */
FA_API const char *fa_status_string(int status);

/* Version of this ABI (bumped when an entry point is added or a signature or
 * a layout changes): 2 = fa_fwd, fa_fwd_kv; 3 adds fa_fwd_splitkv,
 * fa_splitkv_splits and fa_splitkv_workspace_bytes; 4 adds fa_bwd; 5 adds
 * fa_fwd_fp8; 6 adds fa_fwd_splitkv_noalloc. */
FA_API int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
