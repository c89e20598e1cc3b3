/*
 * skinny.h -- C ABI of the weight-only quantized skinny GEMM for MI355X (gfx950).
 *
 *   y[M, N] = x[M, K] . dequant(W)[K, N],   1 <= M <= 8
 *
 * The operation is the one the pages build their decode path on: the
 * weights stay compressed in HBM and each fragment is widened to fp16 in
 * registers right before the matrix unit uses it, with no separate
 * dequantize-to-fp16 pass ("NVFP4 on Volta!" author's post, section "What I
 * actually built").  M = 1 is ordinary decode; M = 8 is the target token
 * plus k = 7 speculative drafts verified in one pass (same post, the
 * paragraph on why the M = 8 row of its bandwidth table matters).  Published
 * FP4 regions go to the NVFP4 path and published FP8 regions to the FP8
 * path, with fp16 activations (same post, section "v1.0 -> v1.1").
 *
 * Formats (OCP MX v1.0 element encodings):
 *   NVFP4 : E2M1 4-bit codes, one E4M3FN scale per 16 consecutive K of one
 *           output column, one fp32 per-tensor scale g.
 *           w~[k][n] = e2m1(q) * e4m3(s) * g
 *   FP8   : E4M3FN codes, one fp32 scale per 128 x 128 block of W.
 *           w~[k][n] = e4m3(c) * S[n/128][k/128]
 *   x     : fp16 (IEEE binary16), row-major [M][K]
 *   y     : fp16, row-major [M][N], round-to-nearest-even of the fp32 sum
 *
 * Conventions shared by every call:
 *   - Every function returns an int status (SKINNY_OK == 0) and never aborts.
 *   - All argument checks happen on the host before any HIP call; a call that
 *     fails them returns an error and enqueues nothing.
 *   - Device pointers must be 16-byte aligned.  The library allocates no
 *     memory: the caller owns every buffer.
 *   - GEMM calls are asynchronous on the caller's stream; faults of the kernel
 *     itself surface at the next synchronisation (HIP semantics).
 *   - Device buffers are passed as bare pointers, so the library cannot check
 *     their sizes or a device blob's header on the host: the caller
 *     guarantees that each buffer holds what the call's shape needs (a blob
 *     packed for exactly this K and N, x of M * K, y of M * N elements).  Any
 *     other buffer gives undefined results and may read out of bounds.  The
 *     Python binding checks these sizes before every call.
 *   - K must be a multiple of 16 (one NVFP4 scale block); N >= 1; K >= 16.
 *   - Results are deterministic: the same inputs give bit-identical outputs.
 */
#ifndef SKINNY_H
#define SKINNY_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  SKINNY_OK = 0,
  SKINNY_EINVAL = 1,   /* null pointer or bad value                          */
  SKINNY_ESHAPE = 2,   /* M, K or N outside what the call supports           */
  SKINNY_EALIGN = 3,   /* device pointer not 16-byte aligned                 */
  SKINNY_ESIZE = 4,    /* output or workspace buffer too small               */
  SKINNY_EHIP = 5,     /* HIP runtime / launch error                         */
  SKINNY_EFORMAT = 6   /* NaN scale byte or bad packed-blob header           */
};

/* Largest supported row count: the target token plus seven drafts. */
#define SKINNY_MAX_M 8

/* Workspaces.  A call that needs one (skinny_workspace_bytes > 0) takes a
 * caller-owned device buffer.  Its first SKINNY_WORKSPACE_SYNC_BYTES bytes
 * hold the arrival counters with which the GEMM kernel adds a K split on
 * each tile group's XCD (the splits of a group run on one XCD and meet in
 * its L2), so they must be zero before the workspace's first use
 * (hipMemset once after allocating); every call leaves them zero, and no call
 * stores anything else there, so one workspace may serve calls of every kind.
 * The rest may hold anything: the call writes every other byte it reads.
 * Calls that share one workspace must not overlap in time. */
#define SKINNY_WORKSPACE_SYNC_BYTES (128u << 10)

/* ---------------------------------------------------------------------------
 * nvfp4_pack -- lay NVFP4 codes and scales out for 128-bit coalesced loads.
 *
 * Host only, run once per weight tensor.  The compressed weights are what the
 * kernels stream from HBM (post, "What I actually built"); this call only
 * reorders bytes, it changes no value.
 *
 *   codes  : host, uint8 [N][K/2]; byte j of row n holds k = 2j in its low
 *            nibble and k = 2j+1 in its high nibble (E2M1 codes).
 *   scales : host, uint8 [N][K/16]; E4M3FN scale of K-block b of column n.
 *            0x7F and 0xFF (NaN) are rejected with SKINNY_EFORMAT.
 *   g      : per-tensor fp32 scale (finite, >= 0).
 *   out    : host buffer of *out_bytes bytes, or NULL to query the size.
 *            On success *out_bytes is set to the blob size.
 *
 * The blob starts with a 256-byte header (magic "SKN4", version 4, K, N, g at
 * byte 28, g again at byte 48, kind 0 at byte 52) followed by 9 KiB units, one per 16 output columns x 1024 K (K padded with
 * zero codes to a multiple of 1024), all tiles of the first K span, then of
 * the next: eight 1 KiB code chunks, then the unit's 1 KiB of scales, ordered
 * so that each lane of a wavefront loads 16 contiguous bytes of every chunk.  The caller copies the
 * blob as-is into a device buffer it owns and passes that to nvfp4_gemm or
 * lm_head_gemm_argmax.  Returns SKINNY_ESIZE if out is non-NULL and
 * *out_bytes is smaller than the blob.
 * ------------------------------------------------------------------------- */
int nvfp4_pack(const uint8_t* codes, const uint8_t* scales, float g,
               int K, int N, void* out, size_t* out_bytes);

/* ---------------------------------------------------------------------------
 * nvfp4_pack_swiglu -- pack the gate and up projections of a gated MLP into
 * one blob for nvfp4_gemm_swiglu.
 *
 * The decode shapes fuse the MLP's gate and up projections into one GEMM
 * over the same x (the fused gate+up shape the post's skinny GEMM serves);
 * the next step of the MLP is h = silu(gate) * up (SwiGLU: Shazeer, "GLU
 * Variants Improve Transformer", 2020).  Packing the pair interleaved lets
 * the GEMM finish that step in registers and write h instead of both
 * projections.
 *
 *   gate_codes, gate_scales, gate_g : canonical NVFP4 arrays of the gate
 *            projection, F output columns (layouts and checks as nvfp4_pack).
 *   up_codes, up_scales, up_g       : the same for the up projection.  The
 *            two scales may differ (one per projection) or be equal (one
 *            scale for the fused tensor).
 *   F      : columns of each projection, 1 .. 2^23.
 *   out, out_bytes : as nvfp4_pack.
 *
 * The blob is an NVFP4 blob of N = 16 * ceil(F / 8) columns: tile t holds
 * gate columns 8t .. 8t+7 as its columns 0..7 and up columns 8t .. 8t+7 as
 * its columns 8..15 (zero weights past F).  Its header has g = gate_g at
 * byte 28, g2 = up_g at byte 48, kind 1 at byte 52 and F at byte 56.
 * ------------------------------------------------------------------------- */
int nvfp4_pack_swiglu(const uint8_t* gate_codes, const uint8_t* gate_scales,
                      float gate_g, const uint8_t* up_codes,
                      const uint8_t* up_scales, float up_g, int K, int F,
                      void* out, size_t* out_bytes);

/* ---------------------------------------------------------------------------
 * nvfp4_gemm -- y = x . (e2m1(q) * e4m3(s) * g), fp32 accumulate, fp16 out.
 *
 *   w_packed  : device, blob from nvfp4_pack for exactly this K and N.
 *   x         : device, fp16 [M][K] row-major.
 *   y         : device, fp16 [M][N] row-major (written, never read).
 *   M         : 1..8.
 *   workspace : device scratch buffer of at least
 *               skinny_workspace_bytes(0, M, K, N) bytes (see "Workspaces":
 *               its first SKINNY_WORKSPACE_SYNC_BYTES zero at rest, the rest
 *               any contents).  May be NULL when that size is 0.  Calls that
 *               share one workspace must not overlap in time.
 *   stream    : HIP stream the kernel is enqueued on (0 = null stream).
 * ------------------------------------------------------------------------- */
int nvfp4_gemm(const void* w_packed, const uint16_t* x, uint16_t* y,
               int M, int K, int N, void* workspace, size_t workspace_bytes,
               hipStream_t stream);

/* ---------------------------------------------------------------------------
 * nvfp4_gemm_noalloc -- nvfp4_gemm for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.
 *
 * Same arguments, layouts, kernel choice and results as nvfp4_gemm (bit for
 * bit), but no workspace: the fp32 partial sums of a K split go to a device
 * array inside the library of SKINNY_NOALLOC_SCRATCH_BYTES (8 MiB), one per
 * GPU, held from the first call on that GPU until the process ends.  The call
 * itself allocates nothing (no hipMalloc, no allocating library routine); the
 * first call on a device looks the array's address up once.
 *   Returns SKINNY_ESIZE, before any HIP call, when the library's kernel
 *   choice for (M, K, N) needs more scratch than that (skinny_workspace_bytes
 *   (0, M, K, N) > SKINNY_NOALLOC_SCRATCH_BYTES); use nvfp4_gemm with a
 *   workspace there.  Other errors as nvfp4_gemm.
 *   Calls that overlap in time on one GPU (two streams, two host threads)
 *   share the array and race; serialize them.  No byte of the array has to
 *   start at any value: every call writes the scratch it reads.
 * ------------------------------------------------------------------------- */
#define SKINNY_NOALLOC_SCRATCH_BYTES (8u << 20)
int nvfp4_gemm_noalloc(const void* w_packed, const uint16_t* x, uint16_t* y,
                       int M, int K, int N, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * nvfp4_gemm_swiglu -- h = silu(x . Wg~) * (x . Wu~), fp16 out.
 *
 *   w_packed  : device, blob from nvfp4_pack_swiglu for exactly this K and F
 *               (the header is in device memory and is not checked; a plain
 *               blob gives meaningless results).
 *   x, M      : as for nvfp4_gemm.
 *   h         : device, fp16 [M][F] row-major (written, never read).
 *   workspace : scratch of at least skinny_workspace_bytes(3, M, K, F) bytes
 *               (as for nvfp4_gemm).
 *
 * Both projections are accumulated in fp32 and scaled by their own g; the
 * activation is applied to those fp32 values in fp32, and only h is rounded
 * to fp16.  The weights are read once, as for nvfp4_gemm.
 * ------------------------------------------------------------------------- */
int nvfp4_gemm_swiglu(const void* w_packed, const uint16_t* x, uint16_t* h,
                      int M, int K, int F, void* workspace,
                      size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * fp8_gemm -- y = x . (e4m3(c) * S), fp32 accumulate, fp16 out.
 *
 * The FP8 regions of a published checkpoint are served in FP8 rather than
 * converted to NVFP4 (post, section "v1.0 -> v1.1").
 *
 *   w            : device, uint8 [N][K] E4M3FN codes (canonical, no packing).
 *   block_scales : device, fp32 [ceil(N/128)][ceil(K/128)].
 *   x, y, M, workspace, stream : as for nvfp4_gemm (op 1 for the size).
 * ------------------------------------------------------------------------- */
int fp8_gemm(const uint8_t* w, const float* block_scales, const uint16_t* x,
             uint16_t* y, int M, int K, int N, void* workspace,
             size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * fp8_pack / fp8_gemm_packed -- the FP8 GEMM on codes reordered once for
 * 128-bit coalesced loads, as nvfp4_pack does for NVFP4 (the codes and their
 * values are unchanged; only the byte order differs).
 *
 * fp8_pack: codes host uint8 [N][K] (K % 16 == 0); out host buffer of
 * *out_bytes bytes, or NULL to query the size.  The blob is a 256-byte header
 * (magic "SKF8", version, K, N) followed by 8 KiB units, one per 16 columns x
 * 512 K (zero codes past K and N), all tiles of the first 512-K span, then
 * of the next, each ordered so that every 16-byte load of a wavefront lane is
 * contiguous with its neighbours' (one KiB per load instruction).  The caller
 * uploads the blob as-is.
 *
 * fp8_gemm_packed: w_packed = that blob in device memory, for exactly this K
 * and N (not checked: device memory); everything else as fp8_gemm, same
 * results bit for bit.
 * ------------------------------------------------------------------------- */
int fp8_pack(const uint8_t* codes, int K, int N, void* out, size_t* out_bytes);
int fp8_gemm_packed(const void* w_packed, const float* block_scales,
                    const uint16_t* x, uint16_t* y, int M, int K, int N,
                    void* workspace, size_t workspace_bytes,
                    hipStream_t stream);

/* ---------------------------------------------------------------------------
 * lm_head_gemm_argmax -- vocabulary-sized NVFP4 GEMM with a fused per-row
 * argmax (post: the native 4-bit lm_head row of the bandwidth table; the
 * drafter should propose greedy / local-argmax tokens, section "This is a
 * server, not a GEMM screenshot").
 *
 *   w_packed, x, M, K, N : as for nvfp4_gemm.
 *   idx       : device, int32 [M]; idx[m] = the smallest n whose fp32 logit
 *               g * sum_k x[m][k] * e2m1 * e4m3 is the row maximum.  The
 *               comparison uses the fp32 logits before any fp16 rounding.
 *   logits    : device fp16 [M][N] or NULL (then no logits are written).
 *   workspace : scratch of at least skinny_workspace_bytes(2, M, K, N) bytes
 *               (as for nvfp4_gemm).
 * ------------------------------------------------------------------------- */
int lm_head_gemm_argmax(const void* w_packed, const uint16_t* x, int32_t* idx,
                        uint16_t* logits, int M, int K, int N, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * lm_head_verify_greedy -- lm_head_gemm_argmax plus the greedy verification
 * of one speculative-decoding round, on the device.
 *
 * A round feeds the target model the last accepted token and k = M - 1 draft
 * tokens d_1 .. d_k; row m of x is its hidden state after token m (row 0:
 * after the last accepted token), so idx[m] is the target's greedy next
 * token there.  Draft d_{j+1} is accepted while it equals idx[j] for every
 * earlier row; with L drafts accepted the round commits d_1 .. d_L and then
 * idx[L], L + 1 tokens (greedy speculative decoding, Leviathan, Kalman and
 * Matias, "Fast Inference from Transformers via Speculative Decoding", 2023;
 * the author's post runs k = 7 native-MTP drafts per round and reports the
 * tokens committed per round, and has the drafter propose greedy tokens).
 *
 *   w_packed, x, M, K, N, workspace : as for lm_head_gemm_argmax (op 2 for
 *               the workspace size).
 *   drafts    : device, int32 [M - 1]: d_1 .. d_{M-1} (may be NULL if M == 1).
 *   idx       : device, int32 [M]: the per-row argmax, as lm_head_gemm_argmax.
 *   result    : device, int32 [M + 1]: result[0] = L (0 .. M-1), result[1 ..
 *               L+1] = the committed tokens, result[L+2 .. M] = -1.
 * The verification runs inside the argmax reduction kernel: no extra launch.
 * ------------------------------------------------------------------------- */
int lm_head_verify_greedy(const void* w_packed, const uint16_t* x,
                          const int32_t* drafts, int32_t* idx, int32_t* result,
                          int M, int K, int N, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Mixed-allocation layer table: each layer of a published checkpoint runs in
 * the precision it was published in, FP4 regions through the NVFP4 path and
 * FP8 regions through the FP8 path, instead of converting the FP8 regions to
 * NVFP4 (post, section "v1.0 -> v1.1": v1.0 served a derived all-NVFP4
 * checkpoint, v1.1 the published mixed allocation).
 *
 *   kind    : SKINNY_LAYER_NVFP4 (nvfp4_gemm), SKINNY_LAYER_FP8 (fp8_gemm),
 *             SKINNY_LAYER_SWIGLU (nvfp4_gemm_swiglu) or
 *             SKINNY_LAYER_FP8_PACKED (fp8_gemm_packed).
 *   weights : device: the packed blob (nvfp4_pack / nvfp4_pack_swiglu /
 *             fp8_pack) or the canonical FP8 codes [N][K].
 *   scales  : device fp32 FP8 block scales; NULL for the NVFP4 kinds.
 *   K, N    : the layer's shape (N = F, the output columns, for a SwiGLU pair).
 * ------------------------------------------------------------------------- */
enum { SKINNY_LAYER_NVFP4 = 0, SKINNY_LAYER_FP8 = 1, SKINNY_LAYER_SWIGLU = 2, SKINNY_LAYER_FP8_PACKED = 3 };

typedef struct skinny_layer {
  int kind;
  const void* weights;
  const float* scales;
  int K, N;
} skinny_layer;

/* Workspace bytes that serve every layer of the table at M rows (the largest
 * single need: the layers run one after another on one stream).  0 if none
 * is needed or a layer is invalid. */
size_t skinny_layers_workspace_bytes(const skinny_layer* layers, int n, int M);

/* Runs layer i on x[i] -> y[i] (device fp16 [M][K_i] -> [M][N_i]) for i = 0 ..
 * n-1, in order on `stream`, each with the library's kernel choice for its
 * kind and shape.  x and y are host arrays of n device pointers; y[i] may be
 * x[i+1] to chain layers.  Every layer is checked before any is enqueued: an
 * invalid one returns its error and nothing runs. */
int skinny_layers_run(const skinny_layer* layers, int n, const uint16_t* const* x,
                      uint16_t* const* y, int M, void* workspace,
                      size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Host quantizers (offline weight preparation, not part of the GEMM).  They
 * stand in for the pages' offline FP16 -> NVFP4 conversion script (ai-manual
 * article, section "NVFP4 model conversion") and produce the canonical
 * arrays that nvfp4_pack and fp8_gemm take.
 *
 * nvfp4_quantize: w host fp32 [K][N] row-major (K % 16 == 0).
 *   g = fp32(amax|w| / 2688); per 16-block of a column: s = E4M3(blk_amax/6/g)
 *   (float64, round to nearest even, saturating); q = E2M1(w / (s*g))
 *   (float64 ratio, RNE, saturating, sign of zero kept; all 0 when s == 0).
 *   Outputs codes [N][K/2], scales [N][K/16] (layouts as nvfp4_pack), *g.
 * fp8_quantize: w host fp32 [K][N]; per 128x128 block S = fp32(blk_amax/448),
 *   c = E4M3(w / S) (float64 ratio; all 0 when S == 0).  Outputs codes [N][K]
 *   and scales [ceil(N/128)][ceil(K/128)].
 * Both reject non-finite weights with SKINNY_EINVAL.
 * ------------------------------------------------------------------------- */
int nvfp4_quantize(const float* w, int K, int N, uint8_t* codes,
                   uint8_t* scales, float* g);
int fp8_quantize(const float* w, int K, int N, uint8_t* codes, float* scales);

/* ---------------------------------------------------------------------------
 * The GEMM calls with an explicit kernel choice instead of the
 * library's pick (same arguments and results, used to compare kernels):
 *   engine : 0 = VALU dot2 engine (nvfp4_gemm, nvfp4_gemm_swiglu,
 *                lm_head_gemm_argmax and lm_head_verify_greedy with M <= 2;
 *                fp8_gemm and fp8_gemm_packed with M <= 4),
 *            1 = MFMA 16x16x32 f16 engine (all calls, M = 1..8),
 *            2 = streaming MFMA engine (nvfp4_gemm and lm_head_gemm_argmax,
 *                K <= 9216): each workgroup keeps all of x in LDS and each
 *                wavefront walks whole column tiles along K, so K is never
 *                split
 *            3 = the VALU engine with one tile of whole K per workgroup,
 *                balanced over the CUs (nvfp4_gemm only, M <= 2; ct = 1,
 *                nw >= the K spans, ksplit = 1).  When the tiles do not
 *                divide evenly over the CUs of the current device and there
 *                are at most four per CU, the tiles past the largest
 *                multiple of the CU count are cut along K into workgroups
 *                of a few spans, at most one per CU, whose partial sums are
 *                added inside the kernel like a K split; every CU then reads
 *                about the same number of weight bytes.  Otherwise it runs
 *                as engine 0.  Needs a workspace (skinny_workspace_bytes_config)
 *   ct     : engines 0, 1: 16-column tiles per workgroup: 1, 2, 4 or 8;
 *            engine 2: workgroups per CU, 1 or 2 (the grid is that many per
 *            CU of the current device, at most 1024)
 *   nw     : wavefronts per workgroup.  Engines 0, 1: ct * S with
 *            S = 1..16/ct: the workgroup covers ct tiles x S consecutive K
 *            spans (1024 K for NVFP4, 512 K for FP8), one span of one tile
 *            per wavefront.  Engine 2: 1..16
 *   ksplit : workgroups that share a tile group along K; with P spans in K
 *            it must satisfy ksplit * S >= P and (ksplit - 1) * S < P
 *            (engine 2: always 1).
 *            With ksplit > 1 each workgroup stores fp32 partial sums in
 *            the workspace (size from skinny_workspace_bytes_config for the
 *            same choice) and they are added in split order: by the last
 *            split to arrive, on the tile group's XCD, for plain NVFP4 calls
 *            on engines 0 and 1 and FP8 calls on engine 1; by a second kernel
 *            otherwise (FP8 on engine 0, SwiGLU pairs, the lm_head).
 * A combination that is not built (or whose LDS need exceeds the CU)
 * returns SKINNY_EINVAL.
 * ------------------------------------------------------------------------- */
int nvfp4_gemm_config(const void* w_packed, const uint16_t* x, uint16_t* y,
                      int M, int K, int N, void* workspace,
                      size_t workspace_bytes, hipStream_t stream, int engine,
                      int ct, int nw, int ksplit);
int fp8_gemm_config(const uint8_t* w, const float* block_scales,
                    const uint16_t* x, uint16_t* y, int M, int K, int N,
                    void* workspace, size_t workspace_bytes, hipStream_t stream,
                    int engine, int ct, int nw, int ksplit);
int fp8_gemm_packed_config(const void* w_packed, const float* block_scales,
                           const uint16_t* x, uint16_t* y, int M, int K, int N,
                           void* workspace, size_t workspace_bytes,
                           hipStream_t stream, int engine, int ct, int nw,
                           int ksplit);
int lm_head_gemm_argmax_config(const void* w_packed, const uint16_t* x,
                               int32_t* idx, uint16_t* logits, int M, int K,
                               int N, void* workspace, size_t workspace_bytes,
                               hipStream_t stream, int engine, int ct, int nw,
                               int ksplit);
int lm_head_verify_greedy_config(const void* w_packed, const uint16_t* x,
                                 const int32_t* drafts, int32_t* idx,
                                 int32_t* result, int M, int K, int N,
                                 void* workspace, size_t workspace_bytes,
                                 hipStream_t stream, int engine, int ct, int nw,
                                 int ksplit);
/* For nvfp4_gemm_swiglu the choice applies to the packed blob's
 * 16 * ceil(F / 8) columns (engine 0 is available for M <= 2). */
int nvfp4_gemm_swiglu_config(const void* w_packed, const uint16_t* x,
                             uint16_t* h, int M, int K, int F, void* workspace,
                             size_t workspace_bytes, hipStream_t stream,
                             int engine, int ct, int nw, int ksplit);

/* 1 if the explicit kernel choice is supported for this op and shape (op as
 * below), else 0. */
int skinny_config_supported(int op, int M, int K, int N, int engine, int ct,
                            int nw, int ksplit);

/* The kernel choice the library makes for a call of this op and shape (op
 * as below), written to *engine, *ct, *nw, *ksplit (host pointers, all
 * non-NULL).  Returns SKINNY_OK, SKINNY_ESHAPE for an unsupported shape or
 * SKINNY_EINVAL for a bad op or NULL pointer.  The choice can be passed to
 * the *_config calls; it is always supported for that op, M and K (the N of
 * another call may make the library choose differently). */
int skinny_default_config(int op, int M, int K, int N, int* engine, int* ct,
                          int* nw, int* ksplit);

/* Workspace bytes of a call made with an explicit kernel choice (op as
 * below); 0 for an unsupported choice or when none is needed. */
size_t skinny_workspace_bytes_config(int op, int M, int K, int N, int engine,
                                     int ct, int nw, int ksplit);

/* Workspace bytes a call needs. op: 0 = nvfp4_gemm, 1 = fp8_gemm,
 * 2 = lm_head_gemm_argmax, 3 = nvfp4_gemm_swiglu (N is then F).  Returns 0
 * for an unsupported op or shape. */
size_t skinny_workspace_bytes(int op, int M, int K, int N);

/* ---------------------------------------------------------------------------
 * skinny_read_probe -- measurement helper, not part of the GEMM path.
 *
 * Reads floor(bytes / 9216) blocks of 9216 bytes of the device buffer `buf`,
 * each by one single-wavefront workgroup with nine 16-byte non-temporal loads
 * per lane (the access shape and cache policy of one NVFP4 unit's loads in
 * the GEMM kernels), and writes nothing else but possibly one word to `sink`
 * (device, 4 bytes).  Timing it gives the HBM read ceiling that the GEMM
 * kernels are rated against (the post, section "What I actually built",
 * rates its kernels against a measured read-only ceiling); of the patterns
 * below it was the fastest at the decode sizes.  Asynchronous on `stream`.
 * SKINNY_ESIZE if bytes < 9216 or the buffer holds 2^31 blocks or more.
 * ------------------------------------------------------------------------- */
int skinny_read_probe(const void* buf, size_t bytes, uint32_t* sink,
                      hipStream_t stream);

/* skinny_read_probe_pattern -- the same probe in other read patterns, to
 * measure which read shape the memory system serves fastest (measurement
 * only).  Reads whole blocks inside [buf, buf + bytes) and writes the number
 * of bytes read to *bytes_read (host pointer, may be NULL).
 *   pattern 0, 1, 2: blocks of 9, 4 or 18 KiB, one per wavefront, all its
 *                    loads issued together; a = wavefronts per workgroup
 *                    (1..16); b unused
 *   pattern 3: the NVFP4 GEMV's shape: 9 KiB units in span-major order of
 *              a K spans (1..16), one workgroup of a wavefronts per tile
 *   pattern 4, 5, 6: a workgroups (1..65535) of b wavefronts (1..16) walk
 *              the 9 KiB blocks with two, three or four blocks in flight per
 *              wavefront
 * SKINNY_EINVAL for a bad pattern, a or b; SKINNY_ESIZE if not one block
 * fits. */
int skinny_read_probe_pattern(const void* buf, size_t bytes, int pattern,
                              int a, int b, uint32_t* sink, size_t* bytes_read,
                              hipStream_t stream);

/* Static description of a status code (never NULL). */
const char* skinny_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* SKINNY_H */
