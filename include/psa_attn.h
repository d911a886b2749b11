/*
 * psa_attn.h — C ABI of libpsa_attn.so: PSA self-attention forward and
 * backward over a conv feature map, for AMD Instinct MI355X (gfx950).
 *
 * The operation (PsaFa2Backward page, vision_rs psa kernels, struct
 * description): Flash-Attention-2 style self-attention in which the query and
 * key sequences are the same N = H*W tokens of one (batch, head) slice and
 * every query attends to every key (no mask, no positional bias).  With
 * Q, K in R^{N x dk}, V in R^{N x dv}, s = scale:
 *
 *   forward   S = s Q K^T,  LSE_i = ln sum_j exp(S_ij),  P = exp(S - LSE),
 *             O = P V
 *   backward  D_i = sum_c dO_ic O_ic,  dS = P o (dO V^T - D),
 *             dQ = s dS K,  dK = s dS^T Q,  dV = P^T dO
 *
 * Layout (same page: packed buffer with sections 0/1/2 = Q/K/V, and the
 * gradient buffer d_packed with sections 0/1/2 = dQ/dK/dV).  Every tensor is
 * dense, contiguous and channel-major, tokens contiguous:
 *   qkv, d_packed  [B, heads, 2*dk + dv, N]   channels [0,dk) Q, [dk,2dk) K,
 *                                             [2dk, 2dk+dv) V
 *   o, dO          [B, heads, dv, N]
 *   lse            [B, heads, N]  float32 in every mode, natural log,
 *                                 scale included
 * Element type of qkv, o, dO and d_packed is given by `dtype`.
 *
 * Pointers are device pointers (hipMalloc'd or equivalent, on the current
 * device) that the caller owns; the library never frees or retains them.
 * Before anything is enqueued, every pointer is looked up with the HIP
 * runtime: host memory, memory of another device, and a tensor whose extent
 * runs past the end of its allocation are refused with PSA_ERR_DEVICE.
 * Base addresses must be 16-byte aligned.  `stream` is a hipStream_t (NULL =
 * the null stream).
 *
 * Calls are asynchronous: they validate, enqueue on `stream` and return.
 * Results are valid once the stream has been synchronised.  On any
 * validation failure nothing is enqueued, nothing is written, a status other
 * than PSA_OK is returned and psa_last_error() describes it.  Faults during
 * execution surface at the caller's next synchronisation.  Outputs are fully
 * overwritten (no zero-initialisation is required).
 *
 * Non-finite inputs are not trapped.  Device code is built in non-IEEE mode
 * (max and min need not propagate NaN), so a NaN or Inf in one (batch, head)
 * slice of the attention inputs leaves that slice's outputs unspecified
 * (they need not be NaN); every other slice's outputs are exactly those of
 * a run without it, as no data passes between slices.
 */
#ifndef PSA_ATTN_H
#define PSA_ATTN_H

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PSA_F32 = 0,  /* float32 storage, float32 arithmetic                    */
  PSA_BF16 = 1, /* bfloat16 storage, bf16 MFMA with float32 accumulation  */
  PSA_F16 = 2   /* IEEE half storage, fp16 MFMA with float32 accumulation */
} psa_dtype_t;

typedef enum {
  PSA_OK = 0,
  PSA_ERR_NULL = 1,        /* a required pointer is NULL                  */
  PSA_ERR_SHAPE = 2,       /* B, heads, N < 1, sizes overflow, bad scale  */
  PSA_ERR_UNSUPPORTED = 3, /* (dk, dv, dtype) has no compiled instance    */
  PSA_ERR_ALIGN = 4,       /* a base pointer is not 16-byte aligned       */
  PSA_ERR_ALIAS = 5,       /* an output overlaps an input or other output */
  PSA_ERR_NOMEM = 6,       /* library scratch could not be allocated      */
  PSA_ERR_HIP = 7,         /* a HIP runtime call or launch failed         */
  PSA_ERR_DEVICE = 8       /* a pointer is not device memory of the
                              current device, or a tensor's extent runs
                              past the end of its allocation              */
} psa_status_t;

/*
 * Forward: O and the row logsumexp LSE from the packed projection.
 *   qkv  in   [B, heads, 2dk+dv, N], dtype
 *   o    out  [B, heads, dv, N], dtype
 *   lse  out  [B, heads, N], float32 (natural log of sum_j exp(s q_i.k_j))
 *   scale     softmax scale s, finite and > 0 (usually 1/sqrt(dk))
 * Scratch: none for float32, or N a multiple of 8, or N < 96.  Otherwise
 * (16-bit rows that 16-byte loads cannot address) qkv is first copied into
 * rows of N8 = N rounded up to 8, zero past N: 2*B*heads*(2dk+dv)*N8 bytes
 * from the per-(device, stream) buffer described under psa_attn_bwd, with
 * the same rules under graph capture.
 */
int psa_attn_fwd(const void* qkv, void* o, float* lse, int B, int heads, int N,
                 int dk, int dv, float scale, int dtype, void* stream);

/*
 * Backward: the packed gradient of sum(dO o O) with respect to qkv.
 *   qkv       in   [B, heads, 2dk+dv, N], dtype
 *   o         in   [B, heads, dv, N], dtype  (D is formed from it as given)
 *   lse       in   [B, heads, N], float32, as written by psa_attn_fwd
 *   dO        in   [B, heads, dv, N], dtype
 *   d_packed  out  [B, heads, 2dk+dv, N], dtype: section 0 = dQ,
 *                  section 1 = dK, section 2 = dV, each element written
 *                  exactly once (deterministic: bitwise identical results
 *                  run to run; no floating-point atomics)
 * Scratch: 8*B*heads*N bytes of device memory from a grow-only buffer the
 * library keeps per (device, stream) until the process ends; the first call
 * on a stream (or a larger one) allocates it with hipMalloc.  For 16-bit
 * rows with N >= 96 not a multiple of 8, qkv, o and dO are first copied
 * into rows of N8 = N rounded up to 8 (zero past N), which adds
 * 2*B*heads*(2dk+2dv)*N8 bytes (each of the four parts rounded up to 256
 * bytes).  Under HIP graph
 * capture: make one uncaptured call of at least the captured size on that
 * stream first (capture cannot allocate), and do not make a larger call on
 * that stream while the graph is in use (growing frees the buffer the graph
 * refers to).
 */
int psa_attn_bwd(const void* qkv, const void* o, const float* lse, const void* dO,
                 void* d_packed, int B, int heads, int N, int dk, int dv, float scale,
                 int dtype, void* stream);

/*
 * psa_attn_bwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments, kernels and results (bitwise identical to
 * psa_attn_bwd; it reads ragged rows in place instead of copying them into
 * padded ones, which changes no bit), but its scratch is a fixed 16 MiB
 * device array compiled
 * into the library, one copy per GPU, held until the process ends.  It
 * calls no hipMalloc, hipFree or other allocating routine.
 * Limit: B*heads*N <= 2097152 (2^21 queries, two fp32 statistics each);
 * larger problems are refused with PSA_ERR_SHAPE before anything is
 * enqueued.  Every call on one GPU shares that GPU's array (its contents
 * are fully rewritten by each call before they are read), so calls that
 * overlap in time on one GPU (concurrent streams or threads) race: order
 * them on one stream.
 */
int psa_attn_bwd_noalloc(const void* qkv, const void* o, const float* lse, const void* dO,
                         void* d_packed, int B, int heads, int N, int dk, int dv, float scale,
                         int dtype, void* stream);

/*
 * The same forward over a slice of V: rows [v0, v0 + dv) of the V section
 * of a packed buffer whose slices hold 2dk + dv_total channels.  This is the
 * call pattern of the PsaFa2Backward page, which runs one attention call per
 * half of V ("lo" and "hi") over the same Q and K; P, and so LSE, are the
 * same for every slice.
 *   qkv  in   [B, heads, 2dk+dv_total, N], dtype
 *   o    out  [B, heads, dv, N], dtype: P V[:, v0:v0+dv]
 *   lse  out  [B, heads, N], float32
 * Requires 0 <= v0 and v0 + dv <= dv_total (else PSA_ERR_SHAPE); (dk, dv)
 * must have a compiled instance.  psa_attn_fwd is the case v0 = 0,
 * dv = dv_total.  Scratch: none.
 */
int psa_attn_fwd_vslice(const void* qkv, void* o, float* lse, int B, int heads, int N, int dk, int dv_total,
                        int v0, int dv, float scale, int dtype, void* stream);

/*
 * The backward of one V-slice call (PsaFa2Backward page: each call owns its
 * V section of d_packed, and the calls share the dQ and dK sections).
 *   qkv, lse   as for psa_attn_fwd_vslice
 *   o, dO      in   [B, heads, dv, N], dtype: this slice's output and its
 *                   upstream gradient (D is formed from them)
 *   d_packed   out  [B, heads, 2dk+dv_total, N], dtype: V rows [v0, v0+dv)
 *                   are overwritten with this slice's dV; the dQ and dK
 *                   sections are overwritten (accumulate = 0) or have this
 *                   slice's dQ and dK added to them (accumulate != 0); other
 *                   V rows are not touched.
 * The page adds the calls' dQ and dK with atomics into zeroed sections; here
 * the first call overwrites and later ones (accumulate = 1) read, add and
 * write each element once, so no zeroing is needed and the result is
 * bitwise reproducible.  Calls that share d_packed must be ordered (one
 * stream): concurrent accumulating calls race.  In 16-bit storage the sum
 * is rounded once per call.  Scratch as for psa_attn_bwd.
 */
int psa_attn_bwd_vslice(const void* qkv, const void* o, const float* lse, const void* dO, void* d_packed, int B,
                        int heads, int N, int dk, int dv_total, int v0, int dv, int accumulate, float scale,
                        int dtype, void* stream);

/*
 * PSA merge (PsaMergeAttnRuntimeOp page: forward and backward of the op
 * that joins the lo and hi attention outputs).  Each head's merged
 * channels are its lo half followed by its hi half:
 *   merged[b][h][c][n] = lo[b][h][c][n],  hi[b][h][c - half][n] for c >= half
 * with lo, hi [B, heads, half, N] and merged [B, heads, 2*half, N] (that is
 * [B, heads*2*half, H, W]), all in dtype.
 * psa_merge_fwd writes merged from (o_lo, o_hi); psa_merge_bwd splits the
 * upstream gradient d_merged into (d_lo, d_hi) by the same map.  Pure
 * copies, no atomics, no scratch; no two of the three tensors may overlap.
 */
int psa_merge_fwd(const void* o_lo, const void* o_hi, void* merged, int B, int heads, int N, int half, int dtype,
                  void* stream);
int psa_merge_bwd(const void* d_merged, void* d_lo, void* d_hi, int B, int heads, int N, int half, int dtype,
                  void* stream);

/*
 * Backward of the 1x1 convolution that produces qkv from the block input x
 * (Conv2dBackward page, struct description, with kh = kw = 1, stride 1, no
 * padding and g = 1; no bias).  The forward is y[b][co][n] = sum_ci
 * w[co][ci] x[b][ci][n]; dy is its upstream gradient, e.g. d_packed of
 * psa_attn_bwd viewed as [B, cout = heads*(2dk+dv), N].
 *   x   in   [B, cin, N], dtype
 *   w   in   [cout, cin], dtype
 *   dy  in   [B, cout, N], dtype
 *   dx  out  [B, cin, N], dtype:  dx[b][ci][n] = sum_co w[co][ci] dy[b][co][n]
 *   dw  out  [cout, cin], dtype:  dw[co][ci] = sum_b sum_n dy[b][co][n] x[b][ci][n]
 * MFMA GEMMs with fp32 accumulation; every output element is written once
 * and the sum over (b, n) for dw runs in a fixed order, so results are
 * bitwise reproducible.  cin and cout must be multiples of 128 (else
 * PSA_ERR_UNSUPPORTED); N is arbitrary.  dx and dw must not overlap the
 * inputs or each other.  Scratch, from the same per-(device, stream)
 * buffer as psa_attn_bwd: when the dw sum is split, S*cout*cin*4 bytes
 * (S <= 64); for 16-bit N not a multiple of 8, zero-padded copies of x and
 * dy with rows of N rounded up to 8 as well (each part rounded up to 256
 * bytes).
 */
int psa_qkv_conv_bwd(const void* x, const void* w, const void* dy, void* dx, void* dw, int B, int cin,
                     int cout, int N, int dtype, void* stream);

/*
 * psa_qkv_conv_bwd for a convolution whose input is a channel concatenation
 * x = cat(x_0, ..., x_{n_parts-1}) along channels, with the concatenation's
 * backward folded into the dx epilogue (ChannelCatBackward page, struct
 * description: the gradient of one concatenated input is its own channel
 * range of the combined gradient).  Part k owns channels [begin_k, begin_k +
 * part_channels[k]) of x, begin_k = part_channels[0] + ... +
 * part_channels[k-1], and receives exactly those rows of dx:
 *   dx_parts[k]  out  [B, part_channels[k], N], dtype:
 *                dx_parts[k][b][c][n] = sum_co w[co][begin_k + c] dy[b][co][n]
 * dx_parts and part_channels are host arrays of n_parts entries (1 <= n_parts
 * <= 4); each part_channels[k] >= 1 and they add up to cin (any split, not
 * only multiples of 128).  x is the concatenated input the forward consumed
 * [B, cin, N]; w, dy, dw, dtype, scratch and determinism are as for
 * psa_qkv_conv_bwd, which is the n_parts = 1 case.  No part may overlap an
 * input, dw or another part; each is 16-byte aligned.
 */
int psa_qkv_conv_cat_bwd(const void* x, const void* w, const void* dy, void* const* dx_parts,
                         const int* part_channels, int n_parts, void* dw, int B, int cin, int cout, int N,
                         int dtype, void* stream);

/*
 * Channel-concatenation backward on its own (ChannelCatBackward page, struct
 * description and index mapping): for the combined gradient dy of a
 * concatenation, one input's gradient is its slice of every outer row,
 *   dx[n * chunk + e] = dy[n * total + offset + e],   n < n_outer, e < chunk.
 * Counts are in elements: for inputs [C_k, H, W] concatenated along channels
 * into [C, H, W] with n_outer = batch, chunk = C_k*H*W, total = C*H*W and
 * offset = (channels before input k)*H*W.
 *   dy  in   [n_outer, total], dtype
 *   dx  out  [n_outer, chunk], dtype; must not overlap dy
 * Requires n_outer, chunk >= 1, offset >= 0, offset + chunk <= total
 * (PSA_ERR_SHAPE otherwise) and 16-byte aligned bases.  A pure copy, no
 * atomics and no scratch; 16-byte vector accesses when chunk, total and
 * offset are multiples of 16 bytes.
 */
int psa_channel_cat_bwd(const void* dy, void* dx, int n_outer, int chunk, int total, int offset, int dtype,
                        void* stream);

/* 1 if (dk, dv, dtype) has a compiled instance, else 0.  No GPU access.
 * Compiled: (dk, dv) in {(32,32), (32,64), (64,32), (64,64), (64,128),
 * (128,128)} for every dtype, and (16,16) for PSA_F32.  (64,32) serves the
 * halves of V at dk = dv = 64 in the V-slice calls. */
int psa_attn_supported(int dk, int dv, int dtype);

/* Message for the last non-OK status returned on the calling thread
 * ("" if none).  The pointer stays valid until the thread's next call. */
const char* psa_last_error(void);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int psa_attn_version(void);

/*
 * Per-kernel device timing, for profiling and roofline reporting.  When
 * enabled, every kernel launch inside the compute entry points is
 * bracketed by two hipEvents recorded on the launch stream; durations are
 * accumulated per kernel.  Off by default; process-wide, thread-safe.
 * Kernel slots: 0 = forward, 1 = backward preprocess (D, LSE*log2 e),
 * 2 = backward GEMM launch (dK/dV and dQ in one grid), 3 = reserved
 * (no kernel; always zero),
 * 4 = psa_qkv_conv_bwd / psa_qkv_conv_cat_bwd dx, 5 = their dw (with its
 * reduction), 6 = psa_channel_cat_bwd, 7 = psa_merge_fwd, 8 = psa_merge_bwd.
 * The V-slice calls use slots 0-3 like psa_attn_fwd / psa_attn_bwd.
 */
#define PSA_TIMING_SLOTS 9
/* on != 0 enables, 0 disables.  Returns PSA_OK. */
int psa_attn_timing_enable(int on);
/* Waits for every recorded launch, then writes min(n, PSA_TIMING_SLOTS)
 * accumulated milliseconds and launch counts (either pointer may be NULL).
 * Returns PSA_OK or PSA_ERR_HIP. */
int psa_attn_timing_read(double* ms, long long* launches, int n);
/* Drops all accumulated and pending measurements.  Returns PSA_OK. */
int psa_attn_timing_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* PSA_ATTN_H */
