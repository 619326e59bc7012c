/*
 * fa.h -- C ABI of libfa: exact scaled-dot-product attention on AMD MI355X
 * (gfx950), computed the IO-aware FlashAttention way.
 *
 * What is computed. For every (batch b, head h), with S = scale * Q K^T:
 *   O   = softmax(S) V                       ("11.11 Flash Attention",
 *                                            section "Standard Attention: Step
 *                                            by Step": the attention formula)
 *   LSE_i = ln sum_j exp(S_ij)               (the per-row statistics m and l of
 *                                            the online softmax, folded into
 *                                            one number, LSE = m + ln l; the
 *                                            zenaique.com page's follow-up on
 *                                            how the backward avoids storing P)
 * The N x N matrices S and P are never written to memory: Q, K and V are
 * tiled on chip and an online softmax keeps a running row max and row sum
 * (same page, sections "Flash Attention: The Key Insight" and "The Tiling
 * Algorithm"); the loop order is Q blocks outer, K/V blocks inner, with the
 * grid parallel over batch x heads x query blocks (section "Flash Attention
 * 2"). The backward recomputes the score tiles from Q, K, V and LSE (section
 * "The Recomputation Trade-off").
 *
 * Conventions shared by every entry point:
 *  - All tensor arguments are DEVICE pointers, allocated and owned by the
 *    caller. The library allocates no memory and keeps no per-call state.
 *  - Layout: contiguous row-major [B, H, N, d] for Q, K, V, O, dO, dQ, dK, dV;
 *    LSE is [B, H, N] float32 (natural log, of the scaled scores).
 *  - Alignment: every [.., N, d] tensor starts on a 16-byte boundary, every
 *    float32 row-statistics array on a 4-byte one (FA_ERR_ARG otherwise).
 *  - d must be 64 or 128 (the 16-bit fa_fwd and fa_bwd also take 256).
 *    B, H, N >= 1, B*H*N*d < 2^31 and B*H*ceil(N/32) < 2^23 (the kernels'
 *    one-dimensional grids stay below 2^32 work-items; the second bound only
 *    matters for sequences of a few tokens). FA_ERR_SHAPE otherwise.
 *  - causal != 0: query i attends to keys 0..i (the mask is not on the pages;
 *    it is the usual lower-triangular mask with N_q = N_k).
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *    and returns without waiting. FA_OK means "launched", not "finished".
 *  - Every argument is validated before anything is launched; on a
 *    validation error (every status except FA_ERR_HIP) nothing is enqueued
 *    and a negative fa_status is returned.
 *  - FA_ERR_HIP reports a failure of this call's own launches: an error left
 *    pending by earlier HIP calls of the same host thread is read and cleared
 *    before the first launch. Entry points that enqueue several kernels
 *    (fa_bwd, fa_bwd_fp8, fa_std_fwd, fa_fwd_splitkv) stop at the first
 *    launch that fails, so the launches before it may already be enqueued;
 *    their outputs are then undefined.
 *  - Calls are thread-safe; calls that share output buffers on one stream are
 *    ordered by the stream.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_F32 = 0,  /* float32 */
    FA_F16 = 1,  /* IEEE half */
    FA_BF16 = 2  /* bfloat16 */
} fa_dtype;

typedef enum {
    FA_OK = 0,
    FA_ERR_NULL = -1,       /* a required pointer is NULL                      */
    FA_ERR_SHAPE = -2,      /* B, H or N < 1, or the tensor is too large         */
    FA_ERR_DTYPE = -3,      /* dtype not supported by this entry point           */
    FA_ERR_HEADDIM = -4,    /* d not supported by this entry point               */
    FA_ERR_WORKSPACE = -5,  /* workspace too small or not 256-byte aligned      */
    FA_ERR_HIP = -6,        /* the HIP runtime reported an error at launch       */
    FA_ERR_ARG = -7,        /* a scalar argument is invalid (scale not finite or
                               not positive, descale not finite or <= 0, split
                               count out of range) or a pointer is misaligned    */
    FA_ERR_TOO_LARGE = -8   /* the problem does not fit the library's fixed
                               scratch (fa_bwd_noalloc only)                    */
} fa_status;

/*
 * Forward pass: O = softmax(scale * Q K^T [causal mask]) V and LSE.
 *   dtype  FA_BF16 / FA_F16: MFMA matrix cores with float32 accumulation, P
 *          rounded to the input type before the P V product, O rounded to
 *          nearest even on store.
 *          FA_F32: float32 arithmetic throughout (no reduced-precision step).
 *   d      64, 128, or (FA_BF16 / FA_F16 only) 256.
 *   q, k, v  [B,H,N,d] of `dtype`, read only.
 *   o        [B,H,N,d] of `dtype`, written.
 *   lse      [B,H,N] float32, written; may be NULL if not wanted.
 *   scale    > 0 and finite; the usual value is 1/sqrt(d).
 */
int fa_fwd(int dtype, const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

/*
 * fa_fwd for 16-bit inputs with the workgroup shape chosen by the caller, for
 * tuning and for measuring the shapes against each other. Each workgroup
 * takes a block of queries ("11.11 Flash Attention", section "Flash
 * Attention 2": parallel over batch, heads and query blocks) and shares the
 * K/V tiles it streams through LDS among its waves:
 *   waves  0: the built-in choice (what fa_fwd runs);
 *          4: four waves, 128 queries per workgroup, two workgroups per CU;
 *          8: eight waves, 256 queries per workgroup, one workgroup per CU
 *             (not at d = 256).
 * Other arguments and errors as fa_fwd (fp32 gives FA_ERR_DTYPE); any other
 * `waves` value gives FA_ERR_ARG. Results are identical for every shape.
 */
int fa_fwd_waves(int dtype, const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int N, int d, float scale, int causal, int waves,
                 hipStream_t stream);

/*
 * FP8 forward ("11.11 Flash Attention", section "Flash Attention 3": FP8
 * attention). Inputs are OCP FP8 E4M3 codes (1 byte each) with one float32
 * descale per tensor: the real value of Q is q8 * q_descale, and likewise for
 * K and V. S = scale * q_descale * k_descale * (Q8 K8^T) is formed by the fp8
 * MFMA with float32 accumulation; the probabilities, taken against a running
 * reference max that trails the row max by at most 2^4 (so p <= 2^4), are
 * scaled by 2^4 and rounded to E4M3 (values <= 256) for the P V product;
 * O is written as bfloat16.
 *   q8, k8, v8  [B,H,N,d] uint8 E4M3 codes, read only.
 *   o_bf16      [B,H,N,d] bfloat16, written.  lse [B,H,N] float32 or NULL.
 *   d must be 128 for this entry point (FA_ERR_HEADDIM otherwise).
 */
int fa_fwd_fp8(const void* q8, const void* k8, const void* v8,
               float q_descale, float k_descale, float v_descale,
               void* o_bf16, float* lse,
               int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

/*
 * Size in bytes of the scratch buffer fa_bwd needs: two float32 vectors of
 * B*H*N entries, the row terms -D_i (D_i = sum_k dO_ik O_ik, stored negated)
 * and LSE_i * log2(e) (each padded to 256 bytes). Returns 0 for invalid
 * shapes.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int N, int d);

/*
 * Backward pass: given dO, returns dQ, dK, dV of L = <O, dO>.
 * The score tiles are recomputed from Q, K and LSE (P_ij = exp(S_ij - LSE_i)),
 * so no N x N matrix is stored ("11.11 Flash Attention", section "The
 * Recomputation Trade-off"). With D_i = sum_k dO_ik O_ik:
 *   dV = P^T dO,  dS = P * (dO V^T - D),  dQ = scale dS K,  dK = scale dS^T Q.
 *   dtype      FA_BF16 or FA_F16 (FA_ERR_DTYPE for FA_F32).
 *   q, k, v, o, dO  [B,H,N,d] of `dtype`; o is the forward output.
 *   lse        [B,H,N] float32 from fa_fwd with the same scale and causal flag.
 *   dq, dk, dv [B,H,N,d] of `dtype`, written.
 *   workspace  device scratch of at least fa_bwd_workspace_bytes(B,H,N,d)
 *              bytes, 256-byte aligned; overwritten (no initial value needed).
 *   d          64, 128 or 256.
 * dK/dV and dQ are produced by two separate passes over the score tiles (no
 * atomics), so all three outputs are bitwise deterministic. At d = 256 the
 * dK/dV pass is two launches (dV, then dK), each recomputing the scores.
 */
int fa_bwd(int dtype, const void* q, const void* k, const void* v, const void* o,
           const float* lse, const void* dO, void* dq, void* dk, void* dv,
           void* workspace, size_t workspace_bytes,
           int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

/*
 * One of the three launches that make up fa_bwd, for callers that time or
 * schedule them separately. Same arguments and validation as fa_bwd, plus
 *   stage 1: -D_i (D_i = sum_k dO_ik O_ik) and LSE_i * log2(e) into the
 *            workspace;
 *   stage 2: per block of keys, recompute P and dS tile by tile and write
 *            dK and dV;
 *   stage 3: per block of queries, recompute P and dS tile by tile and
 *            write dQ.
 * Calling stages 1, 2, 3 in order on one stream is exactly fa_bwd. Stages 2
 * and 3 need stage 1's workspace contents and are independent of each
 * other. Any other stage value returns FA_ERR_ARG.
 */
int fa_bwd_stage(int stage, int dtype, const void* q, const void* k, const void* v,
                 const void* o, const float* lse, const void* dO, void* dq, void* dk, void* dv,
                 void* workspace, size_t workspace_bytes,
                 int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

/*
 * fa_bwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. Same
 * computation, kernels and results (bit for bit) as fa_bwd; the row terms
 * that fa_bwd keeps in the caller's workspace live instead in a scratch
 * array inside the library, one per GPU, 16 MiB, allocated with the library's
 * code object and held until the process ends. Nothing is allocated or freed
 * by the call, and no memset is enqueued (every scratch entry a call reads
 * is first written by that call's own first kernel, so no clearing is
 * needed).
 *   Arguments as fa_bwd, without the workspace. The stream must belong to
 *   the current device (FA_ERR_ARG otherwise); NULL is that device's default
 *   stream.
 *   B*H*N must not exceed fa_bwd_noalloc_max_rows() (2^21): FA_ERR_TOO_LARGE
 *   otherwise, checked before anything is launched.
 * The scratch is shared by every call on one GPU and keeps the last call's
 * contents: calls that overlap in time on one GPU (different streams, or
 * different host threads) race on it and give wrong gradients. Serialise
 * them, e.g. on one stream.
 */
int fa_bwd_noalloc(int dtype, const void* q, const void* k, const void* v, const void* o,
                   const float* lse, const void* dO, void* dq, void* dk, void* dv,
                   int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

/* The largest B*H*N that fa_bwd_noalloc accepts (2^21). */
size_t fa_bwd_noalloc_max_rows(void);

/*
 * Size in bytes of the scratch buffer fa_fwd_splitkv needs for these
 * arguments (same num_splits): the partial outputs (float32,
 * splits x B x H x Nq x d) and partial LSE values of every key range.
 * Returns 0 for invalid arguments.
 */
size_t fa_fwd_splitkv_workspace_bytes(int B, int H, int Nq, int Nk, int d, int num_splits);

/*
 * Forward pass for few queries over many keys (decoding, chunked prefill):
 * the keys are cut into ranges, every (batch, head, 32 queries, key range)
 * is an independent workgroup that writes a normalised partial output and its
 * LSE, and the parts are merged as in fa_lse_merge. Same O and LSE as the
 * definition ("11.11 Flash Attention", section "Flash Attention: The Key
 * Insight": partial softmax results are combined by rescaling with the
 * exponential of the difference of their maxima).
 *   dtype      FA_BF16 or FA_F16.
 *   q, o       [B,H,Nq,d] of `dtype`;  k, v [B,H,Nk,d] of `dtype`.
 *   lse        [B,H,Nq] float32, written; may be NULL.
 *   causal     the queries are the last Nq positions of the Nk keys: query i
 *              sees keys 0 .. Nk - Nq + i (needs Nq <= Nk, else
 *              FA_ERR_SHAPE); Nq = Nk is the square causal mask.
 *   num_splits number of key ranges (1..1024; capped at ceil(Nk / 128)), or
 *              0 to let the library choose about two workgroups per CU.
 *   workspace  at least fa_fwd_splitkv_workspace_bytes(...) bytes, 256-byte
 *              aligned; overwritten.
 * Nq and Nk are any positive sizes with B*H*max(Nq,Nk)*d < 2^31 and
 * B*H*ceil(Nq/32) < 2^23; FA_ERR_SHAPE also if the split grid would reach
 * 2^32 work-items (B*H*ceil(Nq/32)*splits*256).
 */
int fa_fwd_splitkv(int dtype, const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int Nq, int Nk, int d, float scale, int causal, int num_splits,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Merge of attention results over disjoint key sets (the step that joins
 * split key ranges, or the shards of a sequence split across devices): with
 * part p's normalised output O_p and LSE_p = ln sum_{j in part} exp(S_j),
 *   LSE = ln sum_p exp(LSE_p),   O = sum_p exp(LSE_p - LSE) O_p
 * ("11.11 Flash Attention", section "Flash Attention: The Key Insight").
 * A part with LSE_p = -inf has no visible key and is skipped (its O_p is not
 * read); a row whose parts are all empty gets O = 0 and LSE = -inf.
 *   dtype_out  type of o: FA_F32, FA_F16 or FA_BF16.
 *   o_parts    [num_parts][rows][d] float32, 16-byte aligned (FA_ERR_ARG if not).
 *   lse_parts  [num_parts][rows] float32.
 *   o          [rows][d] of dtype_out, written;  lse [rows] float32 or NULL.
 *   d          a multiple of 4 (FA_ERR_SHAPE otherwise); rows * d / 4 at most
 *              2^32 - 256 (one work-item per four output elements).
 */
int fa_lse_merge(int dtype_out, int num_parts, const float* o_parts, const float* lse_parts,
                 void* o, float* lse, int rows, int d, hipStream_t stream);

/*
 * Size in bytes of the scratch buffer fa_fwd_v1 needs: the float32 running
 * output (B*H*N*d) and running max and sum (two copies each per row).
 * Returns 0 for invalid shapes.
 */
size_t fa_fwd_v1_workspace_bytes(int B, int H, int N, int d);

/*
 * Forward pass in the first-generation loop order, for the loop-order
 * ablation ("11.11 Flash Attention", sections "The Tiling Algorithm" and
 * "Flash Attention 2"): one workgroup per (batch, head); the outer loop walks
 * the K/V blocks, the inner loop the Q blocks, and for every block pair the
 * running output O_i (float32) and statistics m_i, l_i are read from and
 * written back to `workspace`, with O renormalised at every step. Same O and
 * LSE as fa_fwd up to rounding; much slower (that is what it measures).
 *   dtype, q, k, v, o, lse, B, H, N, d (64 or 128), scale, causal: as fa_fwd
 *   (16-bit only).
 *   workspace  at least fa_fwd_v1_workspace_bytes(B,H,N,d) bytes, 256-byte
 *              aligned; overwritten.
 */
int fa_fwd_v1(int dtype, const void* q, const void* k, const void* v, void* o, float* lse,
              void* workspace, size_t workspace_bytes, int B, int H, int N, int d, float scale,
              int causal, hipStream_t stream);

/*
 * Size in bytes of the scratch buffer fa_std_fwd needs: the N x N score
 * matrix of every (batch, head) in the 16-bit input type, B*H*N*N*2 bytes
 * (S, then P written over it). Returns 0 for invalid shapes.
 */
size_t fa_std_workspace_bytes(int B, int H, int N, int d);

/*
 * Standard (materialising) attention forward, the baseline the IO-aware path
 * is measured against ("11.11 Flash Attention", section "Standard Attention:
 * Step by Step"): three passes through memory instead of one --
 *   1. S = scale * Q K^T is written to `workspace` (16-bit, [B,H,N,N]);
 *   2. each row is read back and overwritten with P = softmax(S_i) (causal:
 *      P_ij = 0 for j > i);
 *   3. O = P V reads P back.
 * Same O as fa_fwd up to rounding (S and P are rounded to the input type);
 * no LSE. Not the product path: it exists to reproduce the comparison of
 * time and memory that the pages make.
 *   dtype      FA_BF16 or FA_F16.
 *   q, k, v, o [B,H,N,d] of `dtype` as in fa_fwd.
 *   workspace  device scratch of at least fa_std_workspace_bytes(B,H,N,d)
 *              bytes, 256-byte aligned; overwritten.
 * Also FA_ERR_SHAPE if B*H > 65535 or ceil(N/128)^2 * 256 >= 2^32 (grid limits
 * of the score pass).
 */
int fa_std_fwd(int dtype, const void* q, const void* k, const void* v, void* o,
               void* workspace, size_t workspace_bytes,
               int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

/*
 * Size in bytes of the scratch buffer fa_bwd_fp8 needs: bfloat16 copies of
 * the Q, K, V codes plus fa_bwd's own scratch. Returns 0 for invalid shapes.
 */
size_t fa_bwd_fp8_workspace_bytes(int B, int H, int N, int d);

/*
 * Backward pass for fp8 inputs: gradients of L = <O, dO> with respect to the
 * dequantised inputs Q = q_descale * q8 (and likewise K, V), where O and LSE
 * come from fa_fwd_fp8 with the same arguments. The E4M3 codes are widened
 * to bfloat16 (exactly) into the workspace and the 16-bit passes run on the
 * codes with the descales folded into their factors: the exponent uses
 * scale * q_descale * k_descale, the row terms D are divided by v_descale, dK
 * is multiplied by scale * q_descale * v_descale and dQ by
 * scale * k_descale * v_descale ("11.11 Flash Attention", sections "Flash
 * Attention 3" (FP8) and "The Recomputation Trade-off"; the backward
 * equations are those of fa_bwd).
 *   q8, k8, v8      [B,H,N,d] OCP E4M3 codes (uint8), read only.
 *   *_descale       > 0 and finite.
 *   o_bf16, dO_bf16 [B,H,N,d] bfloat16;  lse [B,H,N] float32.
 *   dq, dk, dv      [B,H,N,d] bfloat16, written.
 *   workspace       at least fa_bwd_fp8_workspace_bytes(B,H,N,d) bytes,
 *                   256-byte aligned; overwritten.
 *   d               64, 128 or 256.
 */
int fa_bwd_fp8(const void* q8, const void* k8, const void* v8, float q_descale, float k_descale,
               float v_descale, const void* o_bf16, const float* lse, const void* dO_bf16,
               void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B,
               int H, int N, int d, float scale, int causal, hipStream_t stream);

/*
 * Measurement probe (not part of the attention computation): `blocks`
 * workgroups of four waves each run `iters` rounds of four independent
 * 32x32x16 bf16 MFMAs with operands in registers, i.e. 4 * 4 * iters * 32768
 * FLOP per workgroup, at the chip's practical dense MFMA rate. For each
 * workgroup it writes three values to sink[3*w .. 3*w+2]: elapsed shader
 * clocks (s_memtime), elapsed ticks of the constant-rate real-time counter
 * (s_memrealtime, 100 MHz on this GPU family) and a checksum. The caller
 * times the launch for TFLOP/s; clocks / ticks * 100 MHz is the shader clock
 * under dense MFMA load.
 *   sink    device buffer of 3 * blocks uint64, 8-byte aligned, written.
 *   blocks  1 .. 65536;  iters  1 .. 2^24 (FA_ERR_ARG otherwise).
 */
int fa_probe_mfma(unsigned long long* sink, int blocks, int iters, hipStream_t stream);

/*
 * Measurement probe (not part of the attention computation): the memory side
 * of a one-pass backward, in which the dK/dV pass would also form dQ and add
 * its per-key-block partials into a float32 accumulator with float atomics
 * ("11.11 Flash Attention", section "The Recomputation Trade-off": every
 * (key block, query block) pair contributes to dQ of that query block). For
 * head dim 128 it issues exactly that stream of additions and nothing else:
 * one workgroup per (batch*head, block of key_block keys), placed on the XCDs
 * as the dK/dV pass places its blocks, one 64 x 128 float partial per
 * 64-query step (causal != 0: steps from the key block's first query block
 * on), added with device-scope float atomics (mode 0) or written
 * with plain stores to the same addresses (mode 1). Its duration is a lower
 * bound on what the atomics would add to such a pass.
 *   ws         [B*H*N*128] float32 device buffer, 256-byte aligned; its
 *              contents are accumulated into (mode 0) or overwritten.
 *   N          a multiple of 64 and of key_block;  key_block 128 or 256.
 * FA_ERR_SHAPE / FA_ERR_ARG / FA_ERR_WORKSPACE for arguments outside these.
 */
int fa_probe_dq_atomics(float* ws, size_t ws_bytes, int B, int H, int N, int key_block,
                        int mode, int causal, hipStream_t stream);

/* Human-readable text for a fa_status value (static storage, never NULL). */
const char* fa_status_string(int status);

/* Library ABI version: major * 10000 + minor * 100 + patch. */
int fa_version(void);

/* Build variant flags. FA_BUILD_SERIAL_STAGING is set in the race-guard build
 * (libfa_serial.so), where every kernel that double-buffers its streamed K/V
 * (or Q/dO) tiles in LDS instead keeps one buffer and loads the next tile only
 * once the current one is consumed, so no load overlaps a read. Same
 * arithmetic, same order: its outputs must equal the product build's bit for
 * bit, which tests that the product build's waits and barriers are complete.
 * The guard concerns the tiles that page 2 ("11.11 Flash Attention", section
 * "The Tiling Algorithm") streams through on-chip memory. 0 in libfa.so. */
#define FA_BUILD_SERIAL_STAGING 1
int fa_build_flags(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
