/*
 * sdpa14 -- fused scaled-dot-product attention for AMD MI355X (gfx950).
 *
 * C ABI of libsdpa14.so.  Plain pointers and sizes only; no PyTorch types.
 *
 * The two compute calls follow the forward/backward statement of the nvFuser
 * PR "DID loop split for SDPA" (test test_sdpa_loop_split):
 *
 *   attn, log_sumexp, seed, offset = sdpfa_fwd(q, k, v, dropout_p, is_causal, scale)
 *   q_grad, k_grad, v_grad = sdpfa_bwd(out_grad, q, k, v, attn, log_sumexp,
 *                                      dropout_p, is_causal, seed, offset, scale)
 *
 * What is computed: O = dropout(softmax(Q K^T * scale + causal mask)) V, the
 * definition of scaled-dot-product attention (forum thread
 * "Scaled_dot_product_attention", opening question; nvFuser issue 2278).
 *
 *   - scale: NaN selects 1/sqrt(E).  Otherwise it must be finite and > 0.
 *   - causal: key j is visible to query i iff j <= i (top-left alignment, also
 *     when Sq != Sk).
 *   - log-sum-exp: LSE_i = ln sum_j exp(scale * q_i . k_j) over visible keys, of
 *     the scores before dropout; fp32, contiguous [B, H, Sq].
 *   - dropout: inverted dropout applied to the normalised probabilities: a kept
 *     element is scaled by 1/(1 - p).  The keep bit of element (b, h, i, j) is
 *     Philox-4x32-10 (Salmon et al., SC'11) with key (low, high word of seed)
 *     and counter (low, high word of offset + g, 0, 0), word j % 4, where
 *     g = ((b*H + h)*Sq + i) * ceil(Sk/4) + j/4; kept iff the word is
 *     >= floor(p * 2^32).  The index is absolute, so forward and backward
 *     regenerate the same mask whatever their tiling (PyTorch PR "REDO of
 *     dropout support for mem eff", Summary: RNG state handed from forward to
 *     backward; absolute index for RNG state indexing).
 *   - E == Ev is required (nvFuser issue 2278, the SdpaFwdOp follow-up).
 *   - non-finite inputs follow the definition in the forward: a NaN or an
 *     infinity in query row i makes out row i NaN and LSE row i non-finite
 *     (NaN, or -inf when every score of the row is -inf), and a NaN in key
 *     row j makes NaN the out and LSE rows that can see key j; every other row
 *     is exactly the row of the same call without it.  A NaN in v or dout makes
 *     NaN the outputs whose sums contain it and possibly others (a zero
 *     probability times NaN is NaN inside a tile).
 *
 * Tensors: logical shape [B, H, S, E] with arbitrary element strides for the
 * first three dimensions and unit stride for E.  This covers both stride orders
 * of the nvFuser test: BHSE (memory [b, h, s, e]) and BSHE (memory [b, s, h, e]).
 * Supported now: dtype bf16 or fp16 (IEEE half; one per call); any head dim E
 * that is a multiple of 8 up to 128 (flash kernels commonly take a few fixed
 * head dims; nvFuser issue 2278 notes that Flash Attention does not cover every
 * input, and these calls do not fall back to another path); data pointers
 * 16-byte aligned and the first three strides multiples of 8 elements.  Head
 * dims below 64 run in the head-dim-64 kernels and those between 64 and 128 in
 * the head-dim-128 kernels, with the missing columns read as zeros, so they
 * cost as much as the larger size.
 *
 * Memory: every buffer is owned by the caller and lives on the current HIP
 * device; the library never allocates or frees device memory.  All work is
 * enqueued on `stream` and no call synchronises the device (except
 * sdpa_profile_read).
 *
 * Errors: every compute call returns an sdpa_status.  On a validation error
 * nothing is enqueued, outputs and the RNG state are untouched, and
 * sdpa_last_error() (per thread) describes the problem.  No C++ exception
 * crosses this boundary.  When the HIP runtime refuses a launch the call
 * returns SDPA_ERR_HIP; a forward then takes back its RNG advance (unless
 * another call has moved the state since), because it drew no bits.  For
 * testing that path without a GPU, the environment variable
 * SDPA14_FAIL_LAUNCH (set and not "0", read on every call) makes each compute
 * call return SDPA_ERR_HIP after validation and before any HIP call: nothing
 * is enqueued and the RNG state is untouched.
 *
 * Kernel choices are made per problem.  For comparing them, four variables,
 * read on every call, force one (results are the same within the parity bars;
 * the backward's forms and the two forward orders are bitwise the same):
 * SDPA14_FWD_SHAPE (1: four 32-row sub-tiles, 2: two sub-tiles x two key
 * shares, 3: one sub-tile x four key shares, 4: the causal split launch; a
 * shape the problem cannot take runs as 2), SDPA14_FWD_ORDER (1: the causal
 * split forward in its default workgroup order instead of the host-built
 * dispatch table), SDPA14_BWD_ROLES (1: the backward's two workgroup roles in
 * one launch, 2: in two; two need a call without dropout or bias) and
 * SDPA14_BWD_ORDER (1: the block order computed from the block index instead
 * of the host-built table).
 */
#ifndef SDPA14_H
#define SDPA14_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as hipStream_t; NULL means the default stream. */
typedef struct ihipStream_t* sdpa_stream_t;

typedef enum sdpa_status {
  SDPA_OK = 0,
  SDPA_ERR_INVALID = 1,     /* null pointer, shape mismatch, E != Ev, p not in [0,1), bad scale */
  SDPA_ERR_UNSUPPORTED = 2, /* dtype, head dim, stride or alignment the kernels do not handle */
  SDPA_ERR_WORKSPACE = 3,   /* workspace NULL, misaligned or smaller than required */
  SDPA_ERR_HIP = 4          /* the HIP runtime reported an error at launch */
} sdpa_status;

/* 16-bit element formats; all tensors of one call share one format (the
 * bias too).  Arithmetic is the same for both: 16-bit products into fp32
 * MFMA accumulators, fp32 softmax. */
typedef enum sdpa_dtype { SDPA_BF16 = 0, SDPA_F16 = 1 } sdpa_dtype;

/* A strided device tensor with logical shape [B, H, S, E]. */
typedef struct sdpa_tensor {
  void* data;        /* device pointer, 16-byte aligned */
  int32_t dtype;     /* sdpa_dtype */
  int64_t size[4];   /* B, H, S, E */
  int64_t stride[4]; /* in elements; stride[3] must be 1 */
} sdpa_tensor;

/*
 * Forward (sdpfa_fwd).
 *   q [B,H,Sq,E], k [B,H,Sk,E], v [B,H,Sk,E]  inputs, bf16.
 *   out [B,H,Sq,E]  output, bf16, any supported strides (usually q's).
 *   lse             output, fp32, contiguous [B,H,Sq] (B*H*Sq floats).
 *                   The byte ranges of out and lse (and of keep_bits, see
 *                   sdpa_ext) must not overlap one another or those of q, k, v
 *                   and bias: SDPA_ERR_INVALID.  Inputs may share memory.
 *   seed, offset    host outputs: the Philox state this call used.  When
 *                   dropout_p > 0 the library state's offset then advances by
 *                   B*H*Sq*ceil(Sk/4); when dropout_p == 0 nothing advances
 *                   and no random bits are used.
 */
int sdpa_fwd(const sdpa_tensor* q, const sdpa_tensor* k, const sdpa_tensor* v,
             double dropout_p, int is_causal, double scale,
             const sdpa_tensor* out, float* lse,
             uint64_t* seed, uint64_t* offset, sdpa_stream_t stream);

/*
 * Backward (sdpfa_bwd).
 *   dout, q, k, v, out  bf16 inputs (out and lse as returned by sdpa_fwd).
 *   seed, offset        the values sdpa_fwd returned; ignored when dropout_p == 0.
 *   dq, dk, dv          bf16 outputs shaped like q, k, v (any supported strides);
 *                       their byte ranges must not overlap those of any input
 *                       (SDPA_ERR_INVALID).  They may be views of one packed
 *                       buffer; that their elements are distinct is the
 *                       caller's to ensure.
 *   workspace           device scratch owned by the caller, 256-byte aligned, at
 *                       least sdpa_bwd_workspace_size(B, H, Sq) bytes; it must not
 *                       overlap any tensor and may be reused once the call's work
 *                       on `stream` is done.  Its contents need no initialization.
 * Two kernels run on `stream`: a row pass storing D = rowsum(dO * O) and the
 * row's LSE in base 2 into the workspace, then the main kernel, where dK/dV come
 * from key-block workgroups and dQ from query-block workgroups (no atomics), so
 * all three are bitwise reproducible.
 */
int sdpa_bwd(const sdpa_tensor* dout, const sdpa_tensor* q, const sdpa_tensor* k,
             const sdpa_tensor* v, const sdpa_tensor* out, const float* lse,
             double dropout_p, int is_causal, uint64_t seed, uint64_t offset, double scale,
             const sdpa_tensor* dq, const sdpa_tensor* dk, const sdpa_tensor* dv,
             void* workspace, size_t workspace_bytes, sdpa_stream_t stream);

/*
 * Options of the extended calls (a NULL pointer to them means none).
 *
 *   head_offset, heads_total
 *       Sharding the heads (the nvFuser PR "DID loop split for SDPA" splits the
 *       head dimension over devices and keeps dropout_p = 0 pending sharded
 *       dropout).  The call's head h of batch b is global head head_offset + h
 *       of a problem with heads_total heads (0 means the call's own H), so the
 *       keep bits are those of element (b, head_offset + h, i, j) of the whole
 *       problem: g = ((b*heads_total + head_offset + h)*Sq + i) * ceil(Sk/4) + j/4.
 *       A forward with dropout advances the offset by B*heads_total*Sq*ceil(Sk/4),
 *       as the unsharded call would, so shards stay in step.  Requires
 *       head_offset >= 0, heads_total >= head_offset + H, B*heads_total < 2^31.
 *   rng_state, rng_used  (device pointers to {seed, offset}, 8-byte aligned)
 *       Device-resident RNG state for calls inside a captured HIP graph (the
 *       PyTorch PR "REDO of dropout support for mem eff", Summary: the RNG state
 *       passed from forward to backward so that graph capture works).
 *       Forward: rng_state and rng_used are both given or both NULL, and are
 *       distinct.  When given and dropout_p > 0, a one-thread kernel on `stream`
 *       first copies rng_state to rng_used and advances rng_state's offset by
 *       the amount above; the forward then draws its mask from rng_used.  The
 *       library's host state is neither read nor advanced, and the host outputs
 *       seed and offset are not written.  With dropout_p == 0 nothing is
 *       enqueued for the RNG.  Backward: when rng_used is given, (seed, offset)
 *       are read from it on the device and the host arguments are ignored;
 *       rng_state is ignored.  Both buffers are caller-owned device memory that
 *       must stay valid until the work on `stream` is done.
 *   bias  (NULL for none)
 *       Additive attention bias, the relative-position term the forum thread
 *       "Scaled_dot_product_attention" (opening question) wants SDPA to take
 *       and the attn_bias support the PyTorch PR "REDO of dropout support for
 *       mem eff" announces for the memory-efficient kernel: the scores become
 *       scale * q_i . k_j + bias[b, h, i, j] before masking and softmax, so the
 *       LSE includes it.  Logical shape [B, H, Sq, Sk], bf16, key stride 1,
 *       other strides >= 0 and multiples of 8 elements (0 broadcasts that
 *       dimension), data 16-byte aligned.  Reads go by aligned 8-byte granules,
 *       so the rest of the granule holding a slice's last element is read
 *       (and ignored).  -inf entries hide a key; every row
 *       must keep at least one visible key with a finite score.  Forward and
 *       backward must be given the same bias; dbias below asks for its gradient.
 *   keep_bits  (NULL for none; used only when dropout_p > 0)
 *       Device buffer of sdpa_keep_bits_size(B, H, Sq, Sk) bytes, 16-byte
 *       aligned.  The forward writes the dropout keep bits it draws there (bit
 *       j % 32 of word j / 32 of row (b, h, i), rows of ceil(ceil(Sk/32)/4)*4
 *       words; bits of keys a row cannot see are left unspecified), and a
 *       backward given the same buffer reads them instead of regenerating the
 *       Philox stream in each of its two workgroup roles.  The buffer must
 *       come from the forward with the same inputs, seed and offset, unchanged.
 *   bwd_parts  (backward only; 0 means both)
 *       Which of the backward's two kernels to enqueue: 1 the row pass alone
 *       (D = rowsum(dout * out) and the base-2 LSE into the workspace), 2 the
 *       main kernel alone (dq, dk, dv from a workspace that a row pass of the
 *       same dout, out, lse and scale filled earlier in stream order), 3 or 0
 *       both.  Lets a caller overlap the row pass with other work and time the
 *       two kernels apart; the arguments are validated in full either way.
 *   dbias  (backward only, NULL for none; the forward ignores it)
 *       The bias gradient, for a relative-position term trained through SDPA
 *       (forum thread "Scaled_dot_product_attention", opening question): with
 *       S = scale * q_i . k_j + bias[b, h, i, j], dbias[b, h, i, j] = dL/dS_ij
 *       = P_ij * (dP_ij - D_i), the gradient with respect to the bias as head
 *       (b, h) sees it, and exactly 0 where the causal mask hides the score.
 *       Logical shape [B, H, Sq, Sk], written in full, in q's dtype; key
 *       stride 1, other strides positive multiples of 8 elements with no two
 *       elements sharing memory, data 16-byte aligned, its memory disjoint
 *       from every other argument.  Where the bias broadcasts over a dimension
 *       (stride 0), the caller sums dbias over it: that is the broadcast's own
 *       backward.  Needs bias; written by the main kernel (bwd_parts 2 or 3).
 */
typedef struct sdpa_ext {
  int64_t head_offset;
  int64_t heads_total;
  uint64_t* rng_state;
  uint64_t* rng_used;
  const sdpa_tensor* bias;
  uint32_t* keep_bits;
  int32_t bwd_parts;
  const sdpa_tensor* dbias;
} sdpa_ext;

/* sdpa_fwd / sdpa_bwd with options; sdpa_fwd and sdpa_bwd are these with ext == NULL.
 * sdpa_fwd_ext also accepts lse == NULL: an inference-only forward (the
 * inference node of nvFuser issue 2278) that writes no log-sum-exp, so no
 * backward can follow it. */
int sdpa_fwd_ext(const sdpa_tensor* q, const sdpa_tensor* k, const sdpa_tensor* v,
                 double dropout_p, int is_causal, double scale,
                 const sdpa_tensor* out, float* lse,
                 uint64_t* seed, uint64_t* offset, const sdpa_ext* ext, sdpa_stream_t stream);
int sdpa_bwd_ext(const sdpa_tensor* dout, const sdpa_tensor* q, const sdpa_tensor* k,
                 const sdpa_tensor* v, const sdpa_tensor* out, const float* lse,
                 double dropout_p, int is_causal, uint64_t seed, uint64_t offset, double scale,
                 const sdpa_tensor* dq, const sdpa_tensor* dk, const sdpa_tensor* dv,
                 void* workspace, size_t workspace_bytes, const sdpa_ext* ext,
                 sdpa_stream_t stream);

/*
 * Allocation-free backward, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  The same computation as sdpa_bwd_ext, with the row pass's
 * workspace taken from a fixed scratch array inside the library instead of
 * from the caller: 4 MiB per device, which holds B*H*Sq <= 524288 query rows
 * (sdpa_bwd_noalloc_max_rows()).  Larger problems are rejected with
 * SDPA_ERR_UNSUPPORTED before anything is enqueued.  The call allocates
 * nothing and needs no initialisation: the first call on a device looks up
 * that device's scratch address once.  The caller passes every input and
 * output.  All calls on one device share its scratch and each call
 * overwrites it (nothing in it needs clearing: the row pass writes every row
 * the main kernel reads), so calls whose work overlaps on one device (several
 * streams, several threads) race; serialise them on one stream.
 */
int sdpa_bwd_noalloc(const sdpa_tensor* dout, const sdpa_tensor* q, const sdpa_tensor* k,
                     const sdpa_tensor* v, const sdpa_tensor* out, const float* lse,
                     double dropout_p, int is_causal, uint64_t seed, uint64_t offset,
                     double scale, const sdpa_tensor* dq, const sdpa_tensor* dk,
                     const sdpa_tensor* dv, const sdpa_ext* ext, sdpa_stream_t stream);
/* Largest B*H*Sq sdpa_bwd_noalloc accepts. */
size_t sdpa_bwd_noalloc_max_rows(void);

/* Bytes of the keep-bit cache (sdpa_ext.keep_bits) for a problem; 0 when a size
 * is not positive. */
size_t sdpa_keep_bits_size(int64_t B, int64_t H, int64_t Sq, int64_t Sk);

/* Workspace bytes sdpa_bwd needs for B*H*Sq query rows (8 per row, rounded up to
 * 256); 0 when a size is not positive. */
size_t sdpa_bwd_workspace_size(int64_t B, int64_t H, int64_t Sq);

/* Library-global Philox state (process wide, mutex guarded).  Default (0, 0). */
void sdpa_set_rng_state(uint64_t seed, uint64_t offset);
void sdpa_get_rng_state(uint64_t* seed, uint64_t* offset);

/* Static name of a status code, and the calling thread's last error detail. */
const char* sdpa_status_string(int status);
const char* sdpa_last_error(void);

/*
 * Test hook: writes the dropout keep mask the kernels use, as bytes 0/1, to the
 * device buffer mask [B*H*Sq*Sk] (contiguous b, h, i, j), for the given state
 * and probability.  It uses the same device Philox code as the compute kernels.
 */
int sdpa_debug_dropout_mask(uint64_t seed, uint64_t offset, double dropout_p,
                            int64_t B, int64_t H, int64_t Sq, int64_t Sk,
                            uint8_t* mask, sdpa_stream_t stream);

/*
 * Kernel timing by HIP events, for measurement.  While enabled, every kernel
 * the library launches is bracketed by a pair of events on its own stream
 * (also inside a captured graph: the pairs then time the launches of the
 * latest replay).  sdpa_profile_read waits for the recorded events, returns
 * the summed duration (ms) and launch count of one kernel kind since the last
 * read, and clears that kind.  Kinds: 0 forward kernel, 1 backward main
 * kernel, 2 backward row pass.  At most 8192 launches are kept per kind;
 * further launches are not timed.
 */
enum {
  SDPA_KERNEL_FWD = 0,
  SDPA_KERNEL_BWD = 1,
  SDPA_KERNEL_BWD_ROWS = 2,
  SDPA_KERNEL_KINDS = 3
};
int sdpa_profile_enable(int on);
int sdpa_profile_read(int kind, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* SDPA14_H */
