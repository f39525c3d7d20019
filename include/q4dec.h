/*
 * libq4dec: q4_0 decode hot path for one MI355X (gfx950).
 *
 * The operations follow these pages:
 *  - "visible-cx/gemma-4-E2B-CoreAI" model card: Provenance table (weights are
 *    int4 per-block-32, the ggml q4_0 grid; S=1 decode and S=64 chunked
 *    prefill entry points), the PLE gather-table sidecar section (int8 table,
 *    fp32 per-row scale, multiplier 16.0) and the engine contract (int32 ids,
 *    int8 table, fp32 scale; statics bound over the caller's buffer).
 *  - "Gemma 4 E2B (text decoder) - Core AI" model-zoo card: signature features
 *    (final logit softcap tanh(z/30)*30), "What it took" (fused head with an
 *    in-kernel two-level argmax returning (value, index) with no logit
 *    readback), "QAT weights" (q4_0 = per-block-32 absmax symmetric int4).
 *  - "Gemma-4 E2B mobile mixed-bit QAT weights" knowledge page, P6 section
 *    (stored int4 code = unsigned nibble minus the midpoint 8).
 *
 * Conventions for every call:
 *  - All data pointers are device memory owned by the caller. The library
 *    never allocates, frees, copies to the host or synchronises; each call
 *    validates its arguments on the host, enqueues its kernels on `stream`
 *    (a hipStream_t; NULL means the default stream) and returns. Results are
 *    ready once the caller's stream has been synchronised.
 *  - Return value: Q4DEC_OK (0) on success or a negative Q4DEC_ERR_* code.
 *    Validation errors return before anything is enqueued.
 *    q4dec_last_error() then names the offending argument (thread-local).
 *  - Calls are stateless and thread-safe; the only library state is a cache
 *    of per-device properties (compute-unit count) and the partials array of
 *    lmhead_softcap_argmax_noalloc (see there).
 *  - Activations are bf16 bit patterns (uint16), outputs fp32.
 *  - q4_0 weights enter as unpacked int8 codes c in [-8, 7] plus fp16 scale
 *    bit patterns, one per 32 consecutive weights of a row; q4_pack converts
 *    them into the library's packed layout. The packed layout is opaque and
 *    versioned by Q4DEC_ABI_VERSION; its size is q4_packed_bytes(n, k).
 */
#ifndef Q4DEC_H
#define Q4DEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define Q4DEC_ABI_VERSION 2

#define Q4DEC_OK 0
#define Q4DEC_ERR_NULL -1        /* a required pointer is NULL */
#define Q4DEC_ERR_SHAPE -2       /* n, k, vocab, dim, s or n_ids out of range */
#define Q4DEC_ERR_ALIGN -3       /* pointer misaligned (see each call) */
#define Q4DEC_ERR_WORKSPACE -4   /* workspace smaller than required */
#define Q4DEC_ERR_UNSUPPORTED -5 /* valid request the library does not handle */
#define Q4DEC_ERR_HIP -6         /* HIP runtime error at launch */

/* Largest K (input dimension) the GEMV, head and GEMM kernels accept. */
#define Q4DEC_MAX_K 16384
/* Largest k q4_gemv_gelu_mul handles (the gate/up pairing needs at least two
 * rows per wave step, i.e. at most 32 lanes per row and 6 blocks per lane). */
#define Q4DEC_GELU_MAX_K 6144

/* Library ABI version (Q4DEC_ABI_VERSION of the built library). */
int32_t q4dec_abi_version(void);

/* Text of the last error raised on the calling thread ("" if none). The
 * pointer stays valid until the next failing call on this thread. */
const char* q4dec_last_error(void);

/* Launch-contract checks of a debug build (built with Q4DEC_DEBUG=1; for
 * developers changing the kernels or their plans). Every kernel then first
 * checks that its launch fits what its code assumes (the activation staging
 * holds every block, a plan marked full has no ragged lane, the grid covers
 * every row, tile and K slice); a failed check sets a bit and that workgroup
 * returns before touching memory.
 * q4dec_debug_status synchronises the device, writes the OR of every bit
 * set since the last call to *word (0: no check failed) and clears them.
 * Bits: 0-2 q4_gemv family (staging, full plan, rows), 3-5 per-row kernels,
 * 6-7 multi-vector GEMV (segments, rows), 9-11 S=64 GEMM (chunks, K slices,
 * row tiles), 15 gathers, 17 q4_pack, 18 q4_quantize, 31 self-test.
 * q4dec_debug_selftest launches a kernel whose check always fails (bit 31).
 * Errors: NULL word; Q4DEC_ERR_UNSUPPORTED in a release build (word 0);
 *         Q4DEC_ERR_HIP if the synchronisation reports an error. */
int q4dec_debug_status(uint32_t* word);
int q4dec_debug_selftest(void* stream);

/* Bytes of device memory a packed [n, k] q4_0 matrix occupies: a nibble
 * plane of n*k/2 bytes and an fp16 scale plane of n*(k/32)*2 bytes, each
 * padded to 256 bytes. Returns 0 if n <= 0, k <= 0 or k % 32 != 0. */
size_t q4_packed_bytes(int64_t n, int64_t k);

/* Scale rules of q4_quantize. */
#define Q4DEC_QUANT_Q4_0 0    /* d = m / -8, m the largest-magnitude value; codes in [-8, 7] */
#define Q4DEC_QUANT_ABSMAX7 1 /* d = max|x| / 7; codes in [-7, 7] */

/* q4_quantize: bf16 weights -> q4_0 codes and fp16 block scales, the export
 * step in front of q4_pack (E2B card, QAT weights section: q4_0 is
 * per-block-32 absmax symmetric int4 on the ggml q4_0 grid; the plain absmax
 * variant is the literal grid; model card, Provenance: int4 rounding happens
 * at export). The pages give no formula; per 32-wide block, in fp32:
 *   m   = the value of largest magnitude (lowest index on ties, NaN never),
 *   d   = m / -8 (Q4DEC_QUANT_Q4_0) or max|x| / 7 (Q4DEC_QUANT_ABSMAX7, a
 *         correctly rounded division), stored as fp16 by round to nearest
 *         even (a zero scale is +0),
 *   c_j = clamp(rint(x_j / d16), -8 or -7, 7) with a correctly rounded fp32
 *         quotient and ties to even; c_j = 0 when d16 is 0 or not finite.
 *   x        bf16 [n, k] row-major, 16-byte aligned.
 *   codes    int8 [n, k] row-major output, 16-byte aligned (q4_pack input).
 *   scales   fp16 bit patterns [n, k/32] output, 2-byte aligned.
 *   err_flag optional (NULL allowed) device int32: set to 1 if a block holds
 *            a NaN or its scale overflows fp16; never cleared.
 * Errors: NULL pointer, n <= 0, k <= 0, k % 32 != 0, unknown rule,
 *         misalignment. */
int q4_quantize(const uint16_t* x, int64_t n, int64_t k, int32_t rule,
                int8_t* codes, uint16_t* scales, int32_t* err_flag,
                void* stream);

/* q4_pack: q4_0 codes and scales -> packed layout (load time, not per token).
 *   codes   int8 [n, k] row-major, values in [-8, 7]; stored nibble = c + 8
 *           (mixed-bit page, P6 section).
 *   scales  fp16 bit patterns [n, k/32] row-major; scale b of row r covers
 *           codes[r, 32b .. 32b+31] (model card, Provenance table).
 *   packed  output, q4_packed_bytes(n, k) bytes, 16-byte aligned.
 *   err_flag  optional (NULL allowed) device int32: set to 1 if any code is
 *           outside [-8, 7]; such codes are stored as (c + 8) & 15. Never
 *           cleared by the library.
 * Errors: NULL pointer, n <= 0, k <= 0, k % 32 != 0, packed not 16-aligned. */
int q4_pack(const int8_t* codes, const uint16_t* scales, int64_t n, int64_t k,
            void* packed, int32_t* err_flag, void* stream);

/* q4_gemv: S=1 decode matvec y[r] = sum_k c[r,k] * d[r,k/32] * x[k]
 * (fp32 accumulation; model card Provenance table, S=1 decode). Results are
 * within |y - y_exact| <= 1e-4 * sum_k |w x| + 1e-6 for every finite x: x is
 * staged as fp16 scaled by one power of two per 32-wide block, and when a
 * block's nonzero values span more than 31 binades (a value would lose bits
 * there) the whole call reads x as stored instead (exact path, slower).
 *   packed  from q4_pack with the same (n, k); 16-byte aligned.
 *   x       bf16 [k], 16-byte aligned.
 *   y       fp32 [n], 4-byte aligned; must not overlap packed or x.
 * Errors: NULL pointer, n <= 0, k <= 0, k % 32 != 0, k > Q4DEC_MAX_K,
 *         n >= 2^31, misalignment. */
int q4_gemv(const void* packed, int64_t n, int64_t k, const uint16_t* x,
            float* y, void* stream);

/* q4_gemv_multi: the S=1 matvec for m <= 8 activation vectors at once,
 * y[v, r] = sum_k c[r,k] * d[r,k/32] * x[v, k] (fp32 accumulation), with the
 * weights read once for all m ("Gemma-4 E2B mobile mixed-bit QAT weights",
 * MTP speculative-decoding sections P5c/P5d: one S = 4 verify pass checks four
 * draft rows against weights read once; the FFN and head dominate it).
 * m = 1 is q4_gemv. For m >= 2 the products run on the matrix cores: the
 * vectors are used as stored (bf16) against the codes as exact bf16, so
 * every code-activation product is exact, the products of a block
 * accumulate in fp32 and each block sum is scaled by d in fp32; results are
 * within the q4_gemv bar of the exact sums for every finite x.
 *   packed  from q4_pack with the same (n, k); 16-byte aligned.
 *   x       bf16 [m, k] row-major, 16-byte aligned.
 *   y       fp32 [m, n] row-major, 4-byte aligned, caller-owned.
 * Errors: NULL pointer, n or k as q4_gemv, m not in [1, 8], misalignment;
 *         unsupported when the staged vectors (4 * ceil(m / 4) rows of
 *         (k + 8) bf16 values) do not fit in one workgroup's LDS. */
int q4_gemv_multi(const void* packed, int64_t n, int64_t k, const uint16_t* x,
                  int64_t m, float* y, void* stream);

/* rowq_gemv: per-row symmetric INT8 / INT4 / INT2 matvec on the dense packing
 * of the mixed-bit recipe (mixed-bit page: decode recipe, per-channel
 * symmetric linear weights with all zero points 0; packing convention: INT2
 * holds 4 codes per byte, first code in bits [1:0], two's complement in
 * [-2, 1]; INT4 likewise with nibbles, low nibble first, in [-8, 7]; the
 * INT8 PLE gate / projection matrices are signed bytes; receiving-end
 * design: the integer-weighted sum is scaled once per row):
 *   y[r] = row_scale[r] * sum_k c[r, k] * x[k]   (fp32 accumulation).
 * The raw packed bytes are the kernel's layout (no repacking). Within the
 * q4_gemv bar for every finite x: x is staged per 32-wide block as fp16
 * scaled by a power of two and by the field offset 2^-s the codes are read
 * at (s <= 8 for INT2, 4 for INT4, 0 for INT8); a block whose nonzero values
 * span more than 31 - s binades is summed on its own from x as stored
 * instead (each code * x exact in fp32).
 *   w          [n, k * bits / 8] bytes row-major, 16-byte aligned.
 *   row_scale  fp32 [n], 4-byte aligned.
 *   bits       2, 4 or 8; k a multiple of 64 (INT2) or 32 (INT4, INT8).
 *   x          bf16 [k], 16-byte aligned.   y  fp32 [n], 4-byte aligned.
 * Errors: NULL pointer, bits not 2, 4 or 8, n <= 0 or >= 2^31, k not a
 *         multiple of the code chunk, k > Q4DEC_MAX_K, misalignment. */
int rowq_gemv(const void* w, const float* row_scale, int64_t n, int64_t k,
              int32_t bits, const uint16_t* x, float* y, void* stream);

/* rowq_gemv_gelu_mul: rowq_gemv over the concatenated [gate; up] rows with
 * the fused GELU-tanh * up epilogue (mixed-bit page: the int2 / int4
 * symmetric gate+up kernels run gate, up, GELU and the product in one
 * dispatch). With h = n / 2 and the rowq_gemv sums,
 *   g_j = y[j],  u_j = y[h + j]  (each row with its own scale),
 *   a[j] = RN_bf16(gelu(g_j) * u_j), gelu as in q4_gemv_gelu_mul, j < h.
 *   w, row_scale, bits, x  as rowq_gemv (bits 2, 4 or 8), n rows
 *          ([gate; up]), n even.
 *   a          bf16 bit patterns [n / 2], 2-byte aligned, caller-owned.
 * Errors: those of rowq_gemv, n odd, k > Q4DEC_GELU_MAX_K (unsupported). */
int rowq_gemv_gelu_mul(const void* w, const float* row_scale, int64_t n,
                       int64_t k, int32_t bits, const uint16_t* x,
                       uint16_t* a, void* stream);

/* Workspace bytes rowq_softcap_argmax needs (a fixed 64 KiB: at most 8192
 * per-workgroup partials). */
size_t rowq_head_workspace_bytes(int64_t vocab, int64_t k, int32_t bits);

/* rowq_softcap_argmax: the LM head on the per-row formats (mixed-bit page:
 * the INT2 [262144, 1536] input embedding with its per-row scale is tied
 * with the head; E2B card: the head is fused with its argmax). The logits
 * z[r] are those of rowq_gemv (same kernel, same numerics) and are never
 * written out; the index and capped value of the maximum follow
 * lmhead_softcap_argmax: lowest index among equal maxima, the argmax taken
 * on z, only the winner capped, NaN never wins, idx_out = -1 and
 * val_out = NaN when no logit compares. Two launches on `stream`: each
 * workgroup of the first leaves the best (value, row) of its rows in ws,
 * one workgroup of the second reduces them.
 *   w, row_scale, bits, x  as rowq_gemv with n = vocab.
 *   cap      30.0 for Gemma 4; cap <= 0 returns the raw maximum logit.
 *   ws       device workspace, ws_bytes >= rowq_head_workspace_bytes,
 *            8-byte aligned, caller-owned, no initial contents needed;
 *            calls sharing one ws must not overlap.
 *   idx_out  device int32 [1]; val_out device fp32 [1], 4-byte aligned.
 * Errors: those of rowq_gemv, workspace too small, misalignment. */
int rowq_softcap_argmax(const void* w, const float* row_scale, int64_t vocab,
                        int64_t k, int32_t bits, const uint16_t* x, float cap,
                        void* ws, size_t ws_bytes, int32_t* idx_out,
                        float* val_out, void* stream);

/* q4_gemv_gelu_mul: fused gate/up matvec with the GELU-tanh * up epilogue
 * (mixed-bit page, fused gate/up kernels: one launch over the concatenated
 * [gate; up] rows, fp32 tanh-form GELU in the epilogue). With h = n / 2,
 *   g_j = row j of W . x,  u_j = row h + j of W . x  (fp32 accumulation),
 *   a[j] = RN_bf16(gelu(g_j) * u_j),  gelu(g) = 0.5 g (1 + tanh(sqrt(2/pi)
 *          (g + 0.044715 g^3))) evaluated in fp32,  for j < h.
 * The result is the down projection's bf16 input; no fp32 g or u leaves the
 * kernel. Same weight bytes as q4_gemv on the [n, k] matrix.
 *   packed  from q4_pack of the [gate; up] codes/scales, n rows, n even.
 *   x       bf16 [k], 16-byte aligned.
 *   a       bf16 bit patterns [n / 2], 2-byte aligned, caller-owned.
 * Errors: NULL pointer, n odd or <= 0, k <= 0, k % 32 != 0,
 *         k > Q4DEC_GELU_MAX_K (unsupported), misalignment. */
int q4_gemv_gelu_mul(const void* packed, int64_t n, int64_t k,
                     const uint16_t* x, uint16_t* a, void* stream);

/* Workspace bytes q4_gemm_s64 needs for an [n, k] weight matrix (0 for
 * invalid shapes). */
size_t q4_gemm_workspace_bytes(int64_t n, int64_t k);

/* q4_gemm_s64: chunked-prefill product Y[s, r] = sum_k X[s, k] * w[r, k] for
 * s < n_tok <= 64 (model card, Provenance table: the prefill entry point has a
 * static query width of 64; the weights are read once per 64 tokens). MFMA
 * kernel: per 32-wide block, v_mfma_f32_16x16x32_bf16 multiplies the
 * activations as stored (bf16) by 16 * c (exact in bf16), so every product is
 * exact and each block's sum is formed in fp32; the block sum is then scaled
 * by its fp16 d in fp32 and accumulated, and 1/16 is applied at the end.
 * No activation conversion and no range limit on X short of fp32 overflow:
 * within the q4_gemv bar whenever every |x| < 2^100 (the largest product and
 * block sum then stay finite). Deterministic (fixed summation order). Launches on
 * `stream`: the MFMA kernel and, when K is split over several workgroups,
 * an in-order slice sum.
 *   packed  from q4_pack with the same (n, k); 16-byte aligned.
 *   x       bf16 [n_tok, k] row-major, 16-byte aligned.
 *   y       fp32 [n_tok, n] row-major, 4-byte aligned.
 *   ws      device workspace of ws_bytes >= q4_gemm_workspace_bytes(n, k),
 *           256-byte aligned, caller-owned (split-K partial sums; no initial
 *           contents needed). Calls that share one ws must not overlap.
 * Errors: NULL pointer, n <= 0, k % 32 != 0, k > Q4DEC_MAX_K, n_tok not in
 *         [1, 64], workspace too small, misalignment. */
int q4_gemm_s64(const void* packed, int64_t n, int64_t k, const uint16_t* x,
                int64_t n_tok, float* y, void* ws, size_t ws_bytes,
                void* stream);

/* ---- q4_gemv_chain: one persistent launch over a chain of S=1 GEMVs ----
 * A decode step reads every layer's weights once per token (E4B card,
 * bandwidth cost-model paragraph: bytes per token over the bandwidth plus a
 * fixed per-step cost); with one launch per matrix each of the 169 E4B
 * matrices pays a fixed dispatch cost and starts its weight stream only
 * after the previous kernel has drained (mixed-bit page, fused gate/up
 * paragraph: fewer dispatches per layer help the device). A chain runs its
 * links in one launch: every workgroup walks the links in order, issues the
 * weight loads of its first rows of link i + 1 as soon as it has finished
 * link i, and only then waits (when link i + 1 waits) for every workgroup to
 * finish link i, so the wait runs under the weight stream. Per link the
 * arithmetic is q4_gemv's (and q4_gemv_gelu_mul's, lmhead_softcap_argmax's),
 * with the same results bar. */
#define Q4DEC_LINK_GEMV 0 /* out = fp32 y[n] = W x (q4_gemv) */
#define Q4DEC_LINK_GELU 1 /* out = bf16 a[n/2] (q4_gemv_gelu_mul; k <= Q4DEC_CHAIN_GELU_MAX_K) */
#define Q4DEC_LINK_HEAD 2 /* last link only: softcap + argmax to idx_out / val_out */
#define Q4DEC_CHAIN_MAX_LINKS 4096
#define Q4DEC_CHAIN_MAX_K 10240
#define Q4DEC_CHAIN_GELU_MAX_K 5120

typedef struct q4_chain_link {
  const void* packed;  /* q4_pack output for (n, k); 16-byte aligned */
  const uint16_t* x;   /* bf16 [k], 16-byte aligned; may be an earlier link's output */
  void* out;           /* fp32 [n] (GEMV) or bf16 [n/2] (GELU); unused for HEAD */
  int64_t n, k;
  int32_t mode;        /* Q4DEC_LINK_* */
  int32_t wait;        /* nonzero: stage x only after every workgroup has
                          finished every earlier link (required when x is an
                          earlier link's output) */
} q4_chain_link;

/* Bytes of a chain table for n_links links (0 if n_links is out of range). */
size_t q4_chain_table_bytes(int64_t n_links);

/* Bytes of the chain workspace (error word, arrival counters, head
 * partials). Zero it once before the first call; the kernel leaves it clear
 * after every call that succeeds. */
size_t q4_chain_workspace_bytes(void);

/* q4_chain_build: validates a host array of links and writes the chain table
 * (host memory, q4_chain_table_bytes(n_links) bytes) that q4_gemv_chain
 * runs; the caller copies it once to device memory. Host-only: the links'
 * buffers are not touched. Per link it picks the lane split of the S=1 GEMV.
 * It rejects a chain in which an output shares a 256-byte line with the input
 * of the same or an earlier link or with another link's output, or in which
 * a link reads an earlier output with no waiting link in between (later
 * links read earlier outputs with ordinary cached loads, which is safe only
 * for lines nothing has read before in the launch).
 *   cap      softcap of a head link (30.0; <= 0 disables it).
 *   spin_us  bound on each wait, in microseconds (0: 500000). A wait that
 *            runs out sets the workspace's error word (see q4_gemv_chain).
 *   table    host output, 8-byte aligned.
 * Errors: NULL pointer, n_links out of range, a link's n, k, mode, wait or
 *         alignment invalid (as the matching single-matrix call), k >
 *         Q4DEC_CHAIN_MAX_K, a head link not last, the line rules above,
 *         table too small. */
int q4_chain_build(const q4_chain_link* links, int64_t n_links, float cap,
                   int64_t spin_us, void* table, size_t table_bytes);

/* q4_gemv_chain: runs a built chain as one launch on `stream`: one workgroup
 * of 1024 threads per compute unit, all resident at once (nothing else may
 * occupy the device's compute units while it runs, or its waits run out).
 *   table_host  the table q4_chain_build wrote (checked: tag, checksum).
 *   table_dev   a device copy of it, 64-byte aligned; the kernel checks its
 *               tag, link count and checksum against table_host before use.
 *   ws          q4_chain_workspace_bytes() bytes, 256-byte aligned, zeroed
 *               before the first call and owned by this chain's calls (calls
 *               that share a workspace must not overlap).
 *   idx_out, val_out  device int32 [1] / fp32 [1] for a chain that ends in a
 *               head link (may be NULL otherwise).
 * The first 4 bytes of ws are an error word the kernel sets: 1 when a wait
 * ran out (another workgroup did not arrive in time), 2 when table_dev does
 * not match table_host. While it is nonzero every call returns at once
 * without writing outputs; zero the whole workspace to clear it.
 * Errors: NULL pointer, misalignment, workspace too small, table_host not a
 *         valid built table or built on a device with another compute-unit
 *         count, a head chain without idx_out / val_out. */
int q4_gemv_chain(const void* table_host, const void* table_dev, void* ws,
                  size_t ws_bytes, int32_t* idx_out, float* val_out,
                  void* stream);

/* Workspace bytes lmhead_softcap_argmax needs for a [vocab, k] head. */
size_t lmhead_workspace_bytes(int64_t vocab, int64_t k);

/* lmhead_softcap_argmax: z = W_h x, capped logits cap * tanh(z / cap), and
 * the index and value of their maximum (E2B card: signature features and the
 * fused head + two-level argmax). Lowest index wins among equal maxima. The
 * cap is strictly increasing, so the argmax is taken on z (no per-row tanh)
 * and only the winning value is capped. Logits that are NaN never win; if no
 * logit compares, idx_out = -1 and val_out = NaN. One launch on `stream`:
 * every workgroup publishes its best (value, row) in ws and counts itself
 * in on a counter in ws; the last workgroup to arrive reduces the partials,
 * writes the result and sets the counter back to zero.
 *   packed   from q4_pack with (n = vocab, k); 16-byte aligned.
 *   x        bf16 [k], 16-byte aligned.
 *   cap      30.0 for Gemma 4; cap <= 0 returns the raw maximum logit.
 *   ws       device workspace of ws_bytes >= lmhead_workspace_bytes(vocab, k),
 *            8-byte aligned, owned by the caller: per-workgroup partials,
 *            then the counter. Zero-fill ws once before its first use; every
 *            call leaves the counter at zero. Calls that share one ws must
 *            not overlap (use one stream or separate buffers).
 *   idx_out  device int32 [1]; val_out device fp32 [1].
 * Errors: NULL pointer, vocab <= 0 or >= 2^31, k constraints as q4_gemv,
 *         workspace too small, misalignment. */
int lmhead_softcap_argmax(const void* packed, int64_t vocab, int64_t k,
                          const uint16_t* x, float cap, void* ws,
                          size_t ws_bytes, int32_t* idx_out, float* val_out,
                          void* stream);

/* lmhead_softcap_argmax_noalloc: lmhead_softcap_argmax with no workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc). The
 * per-workgroup partials and the arrival counter live in a device array
 * inside the library: 8192 entries of 8 bytes and one 256-byte line (64.25
 * KiB) on every GPU the library runs on, held until the process ends, zero
 * when the library's code is loaded on the device; every call leaves the
 * counter at zero. The call itself allocates nothing; the first call on a
 * device looks up that array's device address. All calls on one GPU share
 * the array, so calls that overlap in time on one GPU (several streams,
 * several host threads) race and must be serialised by the caller. Same
 * results as lmhead_softcap_argmax (the same kernel).
 *   packed, vocab, k, x, cap, idx_out, val_out  as lmhead_softcap_argmax.
 * Errors: as lmhead_softcap_argmax (no workspace errors);
 *         Q4DEC_ERR_UNSUPPORTED if the head would need more than 8192
 *         workgroup partials; Q4DEC_ERR_HIP if the array's address cannot be
 *         looked up. */
int lmhead_softcap_argmax_noalloc(const void* packed, int64_t vocab, int64_t k,
                                  const uint16_t* x, float cap,
                                  int32_t* idx_out, float* val_out,
                                  void* stream);

/* Workspace bytes lmhead_softcap_argmax_multi needs (m <= 8 vectors). */
size_t lmhead_multi_workspace_bytes(int64_t vocab, int64_t k, int64_t m);

/* lmhead_softcap_argmax_multi: lmhead_softcap_argmax for m <= 8 activation
 * vectors with the head read once ("Gemma-4 E2B mobile mixed-bit QAT
 * weights", MTP sections P5c/P5d: the verify pass reads the head once and
 * takes each draft row's argmax). For each v < m:
 * idx_out[v], val_out[v] as lmhead_softcap_argmax on x[v]; the logits are
 * those of q4_gemv_multi (matrix cores, activations as stored). Two launches on `stream`: the first leaves every workgroup's best
 * (value, row) per vector in ws, the second (one workgroup per vector)
 * reduces them and caps the winner.
 *   packed   from q4_pack with (n = vocab, k); 16-byte aligned.
 *   x        bf16 [m, k] row-major, 16-byte aligned.
 *   ws       device workspace, ws_bytes >= lmhead_multi_workspace_bytes,
 *            8-byte aligned, caller-owned, no initial contents needed; calls
 *            sharing one ws must not overlap.
 *   idx_out  device int32 [m]; val_out device fp32 [m].
 * Errors: as lmhead_softcap_argmax, m not in [1, 8], and unsupported when
 *         the staged vectors (4 * ceil(m / 4) rows of (k + 8) bf16 values)
 *         do not fit in one workgroup's LDS. */
int lmhead_softcap_argmax_multi(const void* packed, int64_t vocab, int64_t k,
                                const uint16_t* x, int64_t m, float cap,
                                void* ws, size_t ws_bytes, int32_t* idx_out,
                                float* val_out, void* stream);

/* Workspace bytes lmhead_softcap_argmax_s64 needs for a [vocab, k] head (0
 * for invalid shapes). */
size_t lmhead_s64_workspace_bytes(int64_t vocab, int64_t k);

/* lmhead_softcap_argmax_s64: the LM head for every row of a prefill chunk of
 * n_tok <= 64 tokens: for each s < n_tok, lmhead_softcap_argmax on x[s]
 * (model card: the prefill entry point has a static query width of 64 and
 * outputs logits for every position; E2B card: the head is fused with its
 * argmax, no logit readback). The logits are those of q4_gemm_s64 (same
 * kernel, same numerics) and are never written out: each workgroup keeps per
 * token the best (logit, row) of its rows. Launches on `stream`: the MFMA
 * kernel, then one workgroup per token reduces the partials and caps the
 * winner.
 *   packed   from q4_pack with (n = vocab, k); 16-byte aligned.
 *   x        bf16 [n_tok, k] row-major, 16-byte aligned.
 *   cap      30.0 for Gemma 4; cap <= 0 returns the raw maximum logits.
 *   ws       device workspace, ws_bytes >= lmhead_s64_workspace_bytes(vocab,
 *            k), 256-byte aligned, caller-owned, no initial contents needed;
 *            calls sharing one ws must not overlap.
 *   idx_out  device int32 [n_tok]; val_out device fp32 [n_tok]; per token as
 *            lmhead_softcap_argmax (lowest row among equal maxima, NaN never
 *            wins, -1 and NaN when no logit compares).
 * Errors: NULL pointer, vocab <= 0 or >= 2^31, k % 32 != 0, k > Q4DEC_MAX_K,
 *         n_tok not in [1, 64], workspace too small, misalignment. */
int lmhead_softcap_argmax_s64(const void* packed, int64_t vocab, int64_t k,
                              const uint16_t* x, int64_t n_tok, float cap,
                              void* ws, size_t ws_bytes, int32_t* idx_out,
                              float* val_out, void* stream);

/* ple_gather: Per-Layer-Embedding row gather
 * out[t, j] = RN_fp32(table[ids[t], j] * row_scale[ids[t]] * mult)
 * (model card, PLE gather-table sidecar section: int8 table [V, L*ld], fp32
 * per-row scale, embed_scale_pl 16.0). The product is rounded once to fp32,
 * so results are bit-identical to the exact product rounded to nearest even.
 *   table      int8 [vocab, dim] row-major.
 *   row_scale  fp32 [vocab].
 *   ids        int32 [n_ids]; an id outside [0, vocab) yields a zero row and
 *              sets *err_flag = 1 (when err_flag is not NULL).
 *   mult       16.0 for the PLE table.
 *   out        fp32 [n_ids, dim] row-major.
 * Errors: NULL pointer (err_flag may be NULL), vocab <= 0, dim <= 0,
 *         n_ids not in [0, 65535] (n_ids == 0 is a no-op), vocab or
 *         dim >= 2^31, row_scale, ids or out not 4-byte aligned. */
int ple_gather(const int8_t* table, const float* row_scale, int64_t vocab,
               int64_t dim, const int32_t* ids, int64_t n_ids, float mult,
               float* out, int32_t* err_flag, void* stream);

/* rowq_gather: row gather on the dense per-row INT2 / INT4 packing of
 * rowq_gemv, with one fp32 scale per group of columns:
 * out[t, j] = RN_fp32(c[ids[t], j] * scales[ids[t], j / group] * mult)
 * (mixed-bit page, bundle table and mixed-bit map: the input embedding, tied
 * with the head, is INT2 [262144, 1536] with one scale per row, group = dim,
 * mult = sqrt(1536); the PLE table stores each row as 35 layer-major
 * 128-byte INT4 blocks with one scale per row and layer, group = 256,
 * mult = 16). The product is rounded once to fp32, as in ple_gather.
 *   w        [vocab, dim * bits / 8] bytes, codes as rowq_gemv (INT2: 4 per
 *            byte, first code in bits [1:0]; INT4: low nibble first; two's
 *            complement); 16-byte aligned.
 *   scales   fp32 [vocab, dim / group].
 *   bits     2 or 4.
 *   group    columns per scale: divides dim, a multiple of 64 (INT2) or 32
 *            (INT4).
 *   ids      int32 [n_ids]; an id outside [0, vocab) yields a zero row and
 *            sets *err_flag = 1 (when err_flag is not NULL).
 *   out      fp32 [n_ids, dim] row-major, 16-byte aligned.
 * Errors: NULL pointer (err_flag may be NULL), bits not 2 or 4, vocab <= 0,
 *         dim not a positive multiple of 64 / 32, group invalid, n_ids not
 *         in [0, 65535], misalignment. */
int rowq_gather(const void* w, const float* scales, int64_t vocab, int64_t dim,
                int32_t bits, int64_t group, const int32_t* ids, int64_t n_ids,
                float mult, float* out, int32_t* err_flag, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* Q4DEC_H */
