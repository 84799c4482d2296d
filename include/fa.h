/*
 * fa.h — C ABI of the MI355X (gfx950) exact-attention library (libfa.so).
 *
 * What the library computes, per (batch b, head h), with Q, K, V, O in
 * R^{N x d} and the softmax scale tau:
 *
 *     S = tau * Q K^T,   S_ij = -inf for j > i when causal,
 *     P = row-wise softmax(S),   O = P V,   LSE_i = ln sum_j exp(S_ij).
 *
 * Definition and causal mask: "FlashAttention 원 논문 해부" (sj-techlog),
 * sections "원 논문의 정의" and "Q·K·V와 한 행의 의미".  The forward is computed
 * tile by tile with per-row online-softmax state (running max, normalizer,
 * unnormalized accumulator) so that S and P never reach device memory:
 * same page, section "두 tile을 한 row로 합치는 식", and "FlashAttention-2:
 * Faster Attention with Better Parallelism and Work Partitioning"
 * (wonbeomjang.kr), section "결과: FlashAttention-2 Forward 알고리즘".  The
 * backward recomputes P from Q, K and the stored LSE (same FlashAttention-2
 * page, sections "개선 2: m과 l 대신 L만 저장" and "Backward Pass").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors q, k, v, o, dout, dq, dk, dv: device pointers to contiguous
 *    [B, H, N, d] arrays of `dtype` (d fastest), 16-byte aligned.
 *  - lse: device pointer to a contiguous [B, H, N] float32 array, natural-log
 *    units (LSE_i = m_i + ln l_i).
 *  - causal != 0: key j is visible to query i iff j <= i (square, top-left
 *    aligned).  Any N >= 1 is accepted; tiles past N are masked.
 *  - scale: the softmax scale tau, used as given (callers usually pass
 *    1/sqrt(d)).  Must be finite.
 *  - Supported: dtype in {FA_F32, FA_F16, FA_BF16}, d in {64, 128}.
 *  - stream: a hipStream_t passed as void* (NULL = the default stream).  All
 *    work is enqueued asynchronously on it; no call synchronizes.
 *  - Ownership: the caller allocates and owns every buffer, the backward
 *    workspace included.  The library allocates no device or host memory and
 *    keeps no state between calls beyond its loaded code objects and a
 *    per-device "is this a gfx950" cache; calls are reentrant.  Inputs must
 *    not alias outputs.
 *  - Errors: a status code, never an exception.  Every argument check runs
 *    before any HIP call; on an argument error nothing is launched and no
 *    output is touched.  Checks: null or misaligned pointers (tensors 16
 *    bytes, lse and cu_seqlens 4 bytes), B/H/N <= 0, element counts
 *    that overflow 64 bits, non-finite scale (FA_ERR_INVALID_ARGUMENT);
 *    unknown dtype, d outside {64, 128}, B or H above 65535, B*H above 2^24,
 *    N above 2^23 or B*H*N above 2^34 (FA_ERR_UNSUPPORTED); workspace
 *    too small or not 256-byte aligned (FA_ERR_WORKSPACE); the current HIP
 *    device is not gfx950 or cannot be queried (FA_ERR_DEVICE); a launch
 *    reported an error (FA_ERR_LAUNCH, outputs then undefined).
 */
#ifndef IO_AWARE_EXACT_FA_AMD_FA_H
#define IO_AWARE_EXACT_FA_AMD_FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_ABI_VERSION 9

/* Block sizes (queries x keys) of the block-sparse mask of fa_attn. */
#define FA_BLOCK_Q 256
#define FA_BLOCK_K 128

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_INVALID_ARGUMENT = 1,
  FA_ERR_UNSUPPORTED = 2,
  FA_ERR_WORKSPACE = 3,
  FA_ERR_DEVICE = 4,
  FA_ERR_LAUNCH = 5
} fa_status;

typedef enum fa_dtype {
  FA_F32 = 0,  /* IEEE binary32 */
  FA_F16 = 1,  /* IEEE binary16 */
  FA_BF16 = 2  /* bfloat16 */
} fa_dtype;

/* Returns FA_ABI_VERSION of the built library. */
int fa_abi_version(void);

/* Returns a static, NUL-terminated description of a status code. */
const char* fa_status_string(fa_status status);

/*
 * Forward pass: o = softmax(scale * q k^T + mask) v and lse, for all B*H heads.
 *
 * Writes every element of o [B,H,N,d] (dtype, rounded to nearest even from
 * the fp32 accumulator after the single division by the row normalizer) and
 * lse [B,H,N] (float32, natural log).  Reads q, k, v.
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int N, int d, int causal, float scale,
                 fa_dtype dtype, void* stream);

/*
 * Bytes of device workspace fa_bwd needs for this shape (0 if the shape is
 * invalid).  With Np = N rounded up to a multiple of 64, the workspace holds
 * two float32 arrays [B,H,Np], 256-byte aligned and in this order:
 *   D   D_i = rowsum(dout_i * o_i)            (rows i >= N: 0)
 *   L2  L2_i = LSE_i * log2(e), the log-sum-exp in base-2 units
 *                                             (rows i >= N: +inf)
 * so that a tile of 64 rows can be copied whole, and P = exp2(S log2(e) - L2)
 * is exactly 0 on padding rows.  Size 2 * 4 * B * H * Np rounded up to 256 B.
 * fa_bwd (and fa_bwd_preprocess) rewrite it completely on every call.  The
 * one-pass steps (fa_bwd_dkdv_dq) need more: this size plus the dQ
 * accumulator, 4 * B * H * Np * d bytes, right after it.
 */
size_t fa_bwd_workspace_size(int B, int H, int N, int d);

/*
 * Backward pass: gradients of sum(O * dout) with respect to q, k, v.
 *
 * o and lse must be what fa_fwd wrote for the same q, k, v, causal and scale.
 * Equivalent to fa_bwd_preprocess, fa_bwd_dkdv and fa_bwd_dq enqueued in that
 * order on `stream` with the same arguments (the two-pass backward: dQ by a
 * separate reduction over the key tiles).  Writes every element of dq, dk, dv
 * (dtype, rounded to nearest even from fp32 accumulators) and of the
 * workspace.  No atomics: results are bitwise repeatable.
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o,
                 const void* dout, const float* lse,
                 void* dq, void* dk, void* dv,
                 int B, int H, int N, int d, int causal, float scale,
                 fa_dtype dtype, void* workspace, size_t workspace_bytes,
                 void* stream);

/*
 * Backward pass for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * fa_bwd without the workspace arguments.  D and L2 (the layout at
 * fa_bwd_workspace_size) go to one static device array of
 * FA_NOALLOC_SCRATCH_BYTES per GPU, part of the library's code object; each
 * GPU the library runs on holds its array until the process ends.  The entry
 * point allocates nothing and calls no allocating routine; on its first call
 * on a device it looks up that device's array address once (the current HIP
 * device must be the one `stream` belongs to).
 *
 * Arguments, results and errors as for fa_bwd, plus: a shape whose
 * fa_bwd_workspace_size exceeds FA_NOALLOC_SCRATCH_BYTES (B * H * Np above
 * 4 Mi rows, Np = N rounded up to 64) is FA_ERR_WORKSPACE, before any launch.
 * Every call on one GPU uses the same array: calls that overlap in time on
 * one GPU (on different streams, or from several threads without ordering)
 * race and give undefined results; calls ordered on one stream are safe.
 * Each call rewrites the array completely, so nothing needs clearing.
 */
#define FA_NOALLOC_SCRATCH_BYTES (32u << 20)

fa_status fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse,
                         void* dq, void* dk, void* dv,
                         int B, int H, int N, int d, int causal, float scale,
                         fa_dtype dtype, void* stream);

/*
 * Backward step 1: D_i = rowsum(dout_i * o_i) and L2_i = LSE_i * log2(e) in
 * float32 into the workspace (layout at fa_bwd_workspace_size); when
 * workspace_bytes also covers the one-pass dQ accumulator
 * (fa_bwd_workspace_size(B, H, N, d) + 4 * B * H * Np * d), it zeroes that
 * too, for fa_bwd_dkdv_dq.  D is the row
 * term of the softmax gradient, precomputed from O instead of from P and dP
 * ("FlashAttention-2: Faster Attention with Better Parallelism and Work
 * Partitioning", sections "Standard Attention Implementation / Backward Pass"
 * and "Backward Pass"); L2 is the stored LSE in the base-2 units the kernels
 * exponentiate in (same page, section "개선 2: m과 l 대신 L만 저장").
 */
fa_status fa_bwd_preprocess(const void* o, const void* dout, const float* lse,
                            int B, int H, int N, int d, fa_dtype dtype,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward step 2: for every tile of keys, recompute P = exp(scale q k^T - lse)
 * query tile by query tile, form dP = dout v^T and dS = P * (dP - D), and write
 * dv = P^T dout and dk = scale * dS^T q (same FlashAttention-2 page, sections
 * "Standard Attention Implementation / Backward Pass" and "Backward Pass": the
 * key/value tile is the outer loop so that one workgroup owns dK_j and dV_j; the
 * factor scale follows from S = scale q k^T by the chain rule).  Needs the
 * workspace as left by fa_bwd_preprocess.
 */
fa_status fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout,
                      const float* lse, void* dk, void* dv,
                      int B, int H, int N, int d, int causal, float scale,
                      fa_dtype dtype, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * Backward step 3: for every tile of queries, recompute P and dS key tile by
 * key tile and write dq = scale * dS k.  This is the separate pass that sums
 * dQ over all key tiles (same FlashAttention-2 page, section "Parallelism:
 * 시퀀스 길이 차원 병렬화", which allows dQ by atomic adds or by a separate
 * reduction).  Needs the workspace as left by fa_bwd_preprocess.  Bitwise
 * repeatable.
 */
fa_status fa_bwd_dq(const void* q, const void* k, const void* v, const void* dout,
                    const float* lse, void* dq,
                    int B, int H, int N, int d, int causal, float scale,
                    fa_dtype dtype, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * One-pass backward, the other reading of the same FlashAttention-2 page
 * (section "Parallelism: 시퀀스 길이 차원 병렬화": dQ by atomic adds instead of a
 * separate reduction).  Step 2 of 3 (after fa_bwd_preprocess with the larger
 * workspace, which zeroes the accumulator): fa_bwd_dkdv (dk and dv written
 * bit for bit the same) that also adds, for every key tile, its share dS k of
 * dQ into the float32 accumulator [B,H,Np,d] that follows D and L2 in the
 * workspace, by atomic adds.  On MI355X it is slower than fa_bwd_dkdv +
 * fa_bwd_dq: the dQ products themselves cost little inside this kernel, but
 * its fp32 atomic adds (B H N d (N / 128) of them) are bound by the L2's
 * atomic rate.  dq then differs in its last bits from call to call (the
 * order of the adds).  k, v, dk, dv have H_kv heads as for the _gqa entry
 * points (H_kv = H: plain heads).  16-bit types only (fp32:
 * FA_ERR_UNSUPPORTED).  workspace_bytes must be at least
 * fa_bwd_workspace_size(B, H, N, d) + 4 * B * H * Np * d.
 */
fa_status fa_bwd_dkdv_dq(const void* q, const void* k, const void* v, const void* dout,
                         const float* lse, void* dk, void* dv,
                         int B, int H, int H_kv, int N, int d, int causal, float scale,
                         fa_dtype dtype, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * One-pass backward, step 3: dq = scale * the accumulator, rounded to dtype
 * (nearest even); rows past N are not read.  16-bit types only; the same
 * workspace size as step 2.
 */
fa_status fa_bwd_dq_finalize(void* dq, int B, int H, int N, int d, float scale,
                             fa_dtype dtype, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * Grouped key/value heads.  The page "Transformer 효율화 기법" (ailab.paldyn.com),
 * section "v1에서 v3까지", lists grouped-query attention (GQA) among the
 * features of FlashAttention-2 without defining it; the reading used here is
 * the usual one: H query heads share H_kv key/value heads (H divisible by
 * H_kv), query head h of a batch entry attends with key/value head
 * h / (H / H_kv) of the same entry; H_kv = 1 is multi-query attention and
 * H_kv = H is plain multi-head attention (the entry points above are exactly
 * these with H_kv = H).  q, o, dout, dq: [B, H, N, d]; k, v, dk, dv:
 * [B, H_kv, N, d]; lse [B, H, N]; the workspace is per query head
 * (fa_bwd_workspace_size(B, H, N, d)) and is filled by fa_bwd_preprocess with
 * H query heads.  dk and dv of a key/value head are the sums of the
 * gradients through all of its query heads (one workgroup walks them in turn,
 * no atomics).  Errors as above; in addition H_kv <= 0 or H not divisible by
 * H_kv is FA_ERR_INVALID_ARGUMENT.
 */
fa_status fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H, int H_kv, int N, int d, int causal, float scale,
                     fa_dtype dtype, void* stream);

fa_status fa_bwd_gqa(const void* q, const void* k, const void* v, const void* o,
                     const void* dout, const float* lse,
                     void* dq, void* dk, void* dv,
                     int B, int H, int H_kv, int N, int d, int causal, float scale,
                     fa_dtype dtype, void* workspace, size_t workspace_bytes,
                     void* stream);

fa_status fa_bwd_dkdv_gqa(const void* q, const void* k, const void* v, const void* dout,
                          const float* lse, void* dk, void* dv,
                          int B, int H, int H_kv, int N, int d, int causal, float scale,
                          fa_dtype dtype, void* workspace, size_t workspace_bytes,
                          void* stream);

fa_status fa_bwd_dq_gqa(const void* q, const void* k, const void* v, const void* dout,
                        const float* lse, void* dq,
                        int B, int H, int H_kv, int N, int d, int causal, float scale,
                        fa_dtype dtype, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * Padding-free variable-length batches.  The 2022 interface described on
 * "FlashAttention 원 논문 해부" (section "내부 구조와 실제 실행 흐름", items 2 and 3)
 * drops padding tokens, packs the valid tokens of all sequences one after
 * another and passes cu_seqlens, the cumulative token offsets, and max_s, the
 * longest length, keeping the softmax statistics per (batch, head, max_s).
 * Sequence b owns the packed rows cu_seqlens[b] <= t < cu_seqlens[b + 1] and
 * attends to its own tokens only (under the causal mask, key j is visible to
 * query i of the same sequence iff j <= i, counted from the sequence's first
 * token).
 *
 *  - q, o, dout, dq: [H, total, d]; k, v, dk, dv: [H_kv, total, d] (dtype, d
 *    fastest, 16-byte aligned): one packed slab per head, so that every
 *    (sequence, head) pair is one contiguous block of rows.  Callers holding
 *    [total, H, d] transpose once.  Grouped heads as for the _gqa entry points.
 *  - cu_seqlens: DEVICE pointer to B + 1 int32 offsets, cu_seqlens[0] = 0,
 *    non-decreasing, every length at most max_s, cu_seqlens[B] <= total.
 *    Read by the kernels, so it cannot be checked before the launch: offsets
 *    outside [0, total] are clamped and lengths cut to max_s, which keeps every
 *    access inside the tensors, but the results are then unspecified.
 *  - lse: [B, H, max_s] float32; entries past a sequence's length are not
 *    written.  Rows of o, dq, dk, dv outside every sequence are not written.
 *  - Empty sequences are allowed (nothing is written for them).
 *  - Workspace: fa_bwd_workspace_size(B, H, max_s, d), same layout as the
 *    dense backward with N = max_s, rewritten by every call.
 *  - Errors as for the dense entry points with N = max_s; in addition
 *    cu_seqlens == NULL or total <= 0 is FA_ERR_INVALID_ARGUMENT.
 */
fa_status fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int* cu_seqlens, int B, int max_s, int total,
                        int H, int H_kv, int d, int causal, float scale,
                        fa_dtype dtype, void* stream);

fa_status fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse,
                        void* dq, void* dk, void* dv,
                        const int* cu_seqlens, int B, int max_s, int total,
                        int H, int H_kv, int d, int causal, float scale,
                        fa_dtype dtype, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * Local windows, and one description of a call for every feature.
 *
 * Local attention keeps, for query i, only the keys j with
 * i - window_left <= j <= i + window_right ("어텐션 비용 줄이기: 희소 어텐션에서
 * FlashAttention과 SSM까지", ailab.paldyn.com, sections "지역 윈도와 글로벌
 * 토큰", w keys on each side, and "슬라이딩 윈도와 수용 영역", the most recent W
 * keys: causal with window_left = W - 1).  Positions count inside each
 * sequence.  Tiles outside every row's window are skipped, so the work and the
 * traffic shrink with the window.  The causal mask still applies when causal
 * != 0 (it acts as window_right = 0).
 *
 * fa_attn fields:
 *   B, H, H_kv, N, d  batch entries (packed: sequences), query heads, key/value
 *                     heads (H_kv divides H), sequence length (packed: max_s),
 *                     head dimension;
 *   causal            as above;
 *   window_left,      >= 0: the window's extent on that side; -1: open.  Every
 *   window_right      row sees at least its own key;
 *   scale, dtype      as above;
 *   cu_seqlens, total NULL for the dense layout [B, H(_kv), N, d]; otherwise a
 *                     packed batch exactly as for fa_fwd_varlen;
 *   dropout_p, seed,  dropout on P (0 <= dropout_p <= 1; 0: none), below.
 *   rng_offset
 *   block_mask,       NULL, or a block-sparse mask, below.
 *   block_mask_heads
 *
 * Block-sparse attention ("FlashAttention 원 논문 해부", section "대안, 비교와
 * 선택 기준": block-sparse FlashAttention skips the zero blocks of a given
 * block mask, so its IO shrinks with the mask's density; it approximates
 * attention by design).  block_mask is a DEVICE array of
 * uint8, [block_mask_heads, ceil(N / FA_BLOCK_Q), ceil(N / FA_BLOCK_K)] row
 * major (N: the sequence length, or max_s of a packed batch); block (qb, kb)
 * covers queries qb FA_BLOCK_Q .. + FA_BLOCK_Q - 1 and keys kb FA_BLOCK_K ..
 * + FA_BLOCK_K - 1 (positions in the sequence), nonzero = computed.
 * block_mask_heads is 1 (one mask for every head) or H (one per query head,
 * shared by the batch entries / sequences).  Key j is visible to query i iff
 * its block is kept and the causal mask and the window allow it; a row that
 * sees no key gets O = 0 and LSE = -inf, and no gradient.  The mask is read by
 * the kernels, which skip the tiles of blocks it drops (the register-staged
 * fp32 kernels and the d = 64 forward test them one by one).  With dropout as
 * well, the dropout applies to P of the kept blocks.
 *
 * Dropout.  The forward computes O = dropout(P) V: element (i, j) of P is kept
 * with probability keep = K / 65536, K = round((1 - dropout_p) 65536), and kept
 * elements are multiplied by 1 / keep; LSE is that of the undropped softmax.
 * The backward regenerates the same mask tile by tile from (seed, rng_offset)
 * ("FlashAttention 원 논문 해부", sections "forward가 끝난 뒤 backward는 무엇을
 * 저장하고 무엇을 다시 계산하는가" and "내부 구조와 실제 실행 흐름": the generator
 * state is kept from the forward, the mask is never stored), so fa_bwd_ex must
 * get the seed, offset and dropout_p of the forward.  The mask: element (i, j)
 * of attention head b H + h (b the sequence of a packed batch, i and j
 * positions in it) is kept iff u < K, u = 16-bit half number (j mod 16) / 2
 * (low half of word 0 first) of Philox4x32-10 (Salmon et al., "Parallel random
 * numbers: as easy as 1, 2, 3", SC 2011) with counter (i, 2 floor(j / 16) +
 * (j mod 2), b H + h, rng_offset) and key (seed mod 2^32, seed / 2^32).  A
 * caller advances rng_offset (or the seed) between steps.
 * Tensors, workspace (fa_bwd_workspace_size(B, H, N, d)), ownership and errors
 * as for the entry points above (dense or packed); in addition p == NULL, a
 * window value below -1, dropout_p outside [0, 1] or block_mask_heads other
 * than 1 or H (with a mask) is FA_ERR_INVALID_ARGUMENT.  fa_bwd_ex needs the o and
 * lse that fa_fwd_ex wrote for the same description.
 */
typedef struct fa_attn {
  int B, H, H_kv, N, d;
  int causal;
  int window_left, window_right;
  float scale;
  fa_dtype dtype;
  const int* cu_seqlens;
  int total;
  float dropout_p;
  unsigned long long seed;
  unsigned int rng_offset;
  const unsigned char* block_mask;
  int block_mask_heads;
} fa_attn;

fa_status fa_fwd_ex(const fa_attn* p, const void* q, const void* k, const void* v, void* o,
                    float* lse, void* stream);

fa_status fa_bwd_ex(const fa_attn* p, const void* q, const void* k, const void* v,
                    const void* o, const void* dout, const float* lse,
                    void* dq, void* dk, void* dv,
                    void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* IO_AWARE_EXACT_FA_AMD_FA_H */
