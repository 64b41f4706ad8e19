/*
 * ssmpack: packed variable-length Mamba-1 sequence operators for MI355X
 * (gfx950). C ABI of libssmpack.so.
 *
 * Pages the operations come from (cited below by tag):
 *   [P5] Shanghai AI Lab HPC/NDS article on packed variable-length Mamba-1
 *        training, https://gitcode.csdn.net/69d8cc1b54b52172bc6872cb.html
 *   [P1] practitioner article on variable-length Mamba-1 training,
 *        https://lpnh.cn/news/2780078
 *   [P3] XTuner variable-length attention guide (Packer, cumulative_len,
 *        position_ids), on pwwt.cn
 *
 * Conventions shared by every entry point:
 *  - Tensors are packed and token-major: a (T, D) tensor holds element
 *    (t, d) at t*D + d, contiguous. T is the total packed token count; a
 *    batch of packs is passed flattened, one cu_seqlens over all of them.
 *  - All tensor pointers are DEVICE pointers (except varlen_pack_plan, a
 *    host function). The caller owns every buffer; the library never
 *    allocates device memory. Workspace sizes are queried first.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL means the
 *    default stream) and returns once its kernels are queued.
 *  - Host-checkable arguments are validated before anything is launched and
 *    reported synchronously as an ssmp_status; nothing is launched then.
 *    Launch failures are reported as SSMP_ERR_HIP. Validity of device-side
 *    cu_seqlens is reported through varlen_pack_indices' dev_err word.
 *  - `dtype` (ssmp_dtype) is the storage type of the (T, D) and (T, N)
 *    tensors. Parameters (A, D skip, conv weight and bias) are always fp32;
 *    so are their gradients and dB, dC. Activation gradients (du, ddelta,
 *    dz, dx) use `dtype`. bf16 results are rounded to nearest even from
 *    fp32 arithmetic; recurrent state and all sums are fp32.
 *  - Gradient buffers are overwritten, never accumulated into.
 */
#ifndef SSMPACK_H
#define SSMPACK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SSMP_OK = 0,
    SSMP_ERR_NULL = 1,        /* a required pointer is NULL */
    SSMP_ERR_SHAPE = 2,       /* a size is out of range, or sizes overflow */
    SSMP_ERR_CU_SEQLENS = 3,  /* cu_seqlens invalid (written to dev_err) */
    SSMP_ERR_UNSUPPORTED = 4, /* dtype, d_state or conv width not supported */
    SSMP_ERR_HIP = 5,         /* a kernel launch failed */
    SSMP_ERR_WORKSPACE = 6,   /* workspace missing or smaller than queried */
    SSMP_ERR_TOO_LARGE = 7    /* needs more than the library's own scratch */
} ssmp_status;

typedef enum { SSMP_F32 = 0, SSMP_BF16 = 1 } ssmp_dtype;

/* Static English text for a status code; never NULL. */
const char *ssmp_status_string(int status);

/* Version of this ABI (incremented on any change to the set of entry points
 * or their meaning; 2 added the _ex scan entry points, 3 the host packer
 * varlen_pack_plan, 4 the scan and conv entry points with sequence states,
 * 5 the scan entry points with a checkpoint interval, 6 the forward scan
 * without allocation). */
int ssmp_abi_version(void);

/*
 * varlen_pack_indices — position_indices from cu_seqlens.
 * [P5] section "conv1d_pack 算子", figure (a): pack() emits, per packed token,
 * its position inside its own sequence (lengths [4,2,3,7] give
 * 0,1,2,3,0,1,0,1,2,0,1,2,3,4,5,6). cu_seqlens follows the FlashAttention
 * varlen convention the article keeps ([P5] "基本原理"; [P3] cumulative_len).
 *
 *   cu_seqlens  device int32 [nseq+1]: cu[0] = 0, non-decreasing,
 *               cu[nseq] = T (zero-length sequences allowed)
 *   pos         device int32 [T] out: pos[t] = t - cu[s] for cu[s] <= t < cu[s+1]
 *   heads       device uint8 [T] out, nullable: 1 where pos[t] == 0, else 0
 *   dev_err     device int32 [1] out, nullable: 0 if cu_seqlens is valid,
 *               else SSMP_ERR_CU_SEQLENS. With an invalid cu_seqlens, pos is
 *               still written in bounds (0 <= pos[t] <= t) but meaningless.
 * Host errors: SSMP_ERR_NULL (cu_seqlens or pos NULL with T > 0),
 * SSMP_ERR_SHAPE (nseq < 1, T < 0, T >= 2^31).
 */
int varlen_pack_indices(const int32_t *cu_seqlens, int32_t nseq, int64_t T,
                        int32_t *pos, uint8_t *heads, int32_t *dev_err, void *stream);

/*
 * conv1d_pack_fwd — causal depthwise conv of width W that stops at each
 * sequence's head token, then optional SiLU.
 * [P5] "conv1d_pack 算子": the conv looks back W-1 tokens and terminates
 * early at a head; [P1] 2.2: no tap may cross a document boundary.
 *   u[t,d] = act(b[d] + sum_{k=0}^{min(pos[t],W-1)} w[d,W-1-k] * x[t-k,d])
 * with act = SiLU if silu != 0, identity otherwise.
 *   x    (T, D) dtype          w  fp32 (D, W); w[d,W-1] multiplies token t
 *   b    fp32 (D), nullable    pos int32 (T) from varlen_pack_indices
 *   u    (T, D) dtype out
 * Supports 1 <= W <= 4. Taps k > t are never read, whatever pos holds.
 * Errors: SSMP_ERR_NULL, SSMP_ERR_SHAPE (T < 0, D < 1, T*D >= 2^40),
 * SSMP_ERR_UNSUPPORTED (W outside 1..4, unknown dtype).
 */
int conv1d_pack_fwd(const void *x, const float *w, const float *b, const int32_t *pos, void *u,
                    int64_t T, int32_t D, int32_t W, int32_t dtype, int32_t silu, void *stream);

/*
 * conv1d_pack_bwd — gradients of conv1d_pack_fwd given du = dL/du.
 * [P5] "conv1d_pack 算子": dx and dweight stop early too; the reverse position
 * comes from pos W-1 tokens ahead: token s receives from s+k only if
 * pos[s+k] >= k.
 *   dx (T, D) dtype out;  dw fp32 (D, W) out;  db fp32 (D) out, nullable
 * workspace: device memory of at least conv1d_pack_bwd_workspace_bytes(T, D, W)
 * bytes (per-tile partial sums of dw and db; contents need not be
 * initialised). Sums over tokens are deterministic (fixed order).
 * Errors as conv1d_pack_fwd, plus SSMP_ERR_WORKSPACE.
 */
size_t conv1d_pack_bwd_workspace_bytes(int64_t T, int32_t D, int32_t W);
int conv1d_pack_bwd(const void *x, const float *w, const float *b, const int32_t *pos,
                    const void *du, void *dx, float *dw, float *db,
                    void *workspace, size_t workspace_bytes,
                    int64_t T, int32_t D, int32_t W, int32_t dtype, int32_t silu, void *stream);

/*
 * conv1d_pack_fwd_states / conv1d_pack_bwd_states — the conv with a context
 * per sequence: the W-1 inputs that precede a sequence's first token, which
 * the reset otherwise treats as zeros. [P5] "结论与讨论" (a sequence cut at a
 * pack end continues in the next pack) and [P1] section 3.2 (segment runs
 * that reset or pass conv_states). With cu_seqlens (device int32 [nseq+1],
 * the one pos was built from):
 *   conv_initial   dtype (nseq, W-1, D), nullable (zeros): the context of
 *                  sequence s, element (s, j, d) at (s*(W-1) + j)*D + d,
 *                  j = 0 the oldest input, j = W-2 the one just before the
 *                  sequence's first token
 *   conv_final     dtype (nseq, W-1, D) out, nullable: the context a sequence
 *                  hands on, its own last W-1 inputs (reaching into its
 *                  context when shorter than W-1)
 *   dconv_final    dtype (nseq, W-1, D), nullable (zero): dL/d conv_final
 *   dconv_initial  dtype (nseq, W-1, D) out, nullable: dL/d conv_initial
 * A piece that continues a sequence takes the previous piece's conv_final as
 * its conv_initial (and the previous piece's backward takes this piece's
 * dconv_initial as its dconv_final). The backward needs
 * conv1d_pack_bwd_states_workspace_bytes(T, D, W, nseq) bytes of workspace
 * (per-sequence corrections join the fixed-order sums). State buffers must
 * not overlap one another or x, u, du, dx. With every state pointer NULL
 * these are conv1d_pack_fwd / conv1d_pack_bwd.
 * Errors as conv1d_pack_fwd / _bwd, plus SSMP_ERR_NULL (a state pointer
 * without cu_seqlens) and SSMP_ERR_SHAPE (nseq < 1 with a state pointer).
 */
int conv1d_pack_fwd_states(const void *x, const float *w, const float *b, const int32_t *pos, void *u,
                           int64_t T, int32_t D, int32_t W, int32_t dtype, int32_t silu,
                           const int32_t *cu_seqlens, int32_t nseq, const void *conv_initial,
                           void *conv_final, void *stream);
size_t conv1d_pack_bwd_states_workspace_bytes(int64_t T, int32_t D, int32_t W, int32_t nseq);
int conv1d_pack_bwd_states(const void *x, const float *w, const float *b, const int32_t *pos,
                           const void *du, void *dx, float *dw, float *db,
                           void *workspace, size_t workspace_bytes,
                           int64_t T, int32_t D, int32_t W, int32_t dtype, int32_t silu,
                           const int32_t *cu_seqlens, int32_t nseq, const void *conv_initial,
                           const void *dconv_final, void *dconv_initial, void *stream);

/*
 * selective_scan_pack_fwd — the selective scan with the state reset to zero
 * at every head token ([P5] "SSM_pack算子" and "基本原理": the state flows
 * across packed sequences only through the recurrence, so it is reset at
 * each boundary). Per channel d and state n:
 *   h_t = exp(delta_t A[d,n]) h_{t-1} + delta_t B_t[n] u_t   (h_{t-1} = 0 at a head)
 *   y_t = sum_n C_t[n] h_t[n] + Dskip[d] u_t
 *   out_t = y_t * SiLU(z_t)                                   (out = y if z is NULL)
 *   u, delta, z, out  (T, D) dtype;  B, C (T, N) dtype (shared by all channels)
 *   A  fp32 (D, N);  Dskip fp32 (D), nullable;  pos int32 (T)
 *   delta is used as given (already positive).
 * workspace: device memory of selective_scan_pack_workspace_bytes(T, D, N)
 * bytes. The forward writes fp32 state checkpoints into it that
 * selective_scan_pack_bwd reads; keep it untouched between the two calls,
 * and pass the backward the same inputs.
 * Supports N in {1, 2, 4, 8, 16}.
 * Errors: SSMP_ERR_NULL, SSMP_ERR_SHAPE, SSMP_ERR_UNSUPPORTED, SSMP_ERR_WORKSPACE.
 */
size_t selective_scan_pack_workspace_bytes(int64_t T, int32_t D, int32_t N);
int selective_scan_pack_fwd(const void *u, const void *delta, const float *A, const void *B,
                            const void *C, const float *Dskip, const void *z, const int32_t *pos,
                            void *out, void *workspace, size_t workspace_bytes,
                            int64_t T, int32_t D, int32_t N, int32_t dtype, void *stream);

/*
 * selective_scan_pack_bwd — gradients of selective_scan_pack_fwd given
 * dout = dL/dout, by a reverse scan whose carry is cut at every head (no
 * gradient crosses a sequence boundary).
 *   du, ddelta (T, D) dtype out
 *   dA fp32 (D, N) out; dB, dC fp32 (T, N) out (sums over channels)
 *   dD fp32 (D) out, nullable (must be NULL iff Dskip is NULL)
 *   dz (T, D) dtype out, nullable (must be NULL iff z is NULL)
 * The workspace must hold the forward's checkpoints (same inputs, same
 * workspace, no call on it in between). Sums over tokens and channels are
 * deterministic.
 * Errors as selective_scan_pack_fwd.
 */
int selective_scan_pack_bwd(const void *u, const void *delta, const float *A, const void *B,
                            const void *C, const float *Dskip, const void *z, const int32_t *pos,
                            const void *dout, void *workspace, size_t workspace_bytes,
                            void *du, void *ddelta, float *dA, float *dB, float *dC,
                            float *dD, void *dz,
                            int64_t T, int32_t D, int32_t N, int32_t dtype, void *stream);

/*
 * selective_scan_pack_fwd_ex / selective_scan_pack_bwd_ex — the same scan with
 * two element-wise neighbours applied where it reads its inputs:
 *   - the step map: the scan uses softplus(delta + delta_bias[d]) (when
 *     delta_softplus is nonzero) or delta + delta_bias[d] in place of delta.
 *     delta_bias is fp32 (D), nullable (no bias). The pages take the step as
 *     given; this is Mamba-1's discretisation step, bias and softplus folded
 *     in so that no separate (T, D) pass produces it.
 *   - the gate floor: out = y * (SiLU(z) + gate_floor), [P4]
 *     (aimodeling.com, near-zero embeddings in gated training) "修法"
 *     GateFloor, a positive offset (there 0.01 .. 0.1) that keeps the gate
 *     above zero at zero input. 0 is the plain SiLU gate; ignored without z.
 * The backward returns ddelta with respect to the stored delta (times
 * sigmoid(delta + bias) under softplus) and ddelta_bias fp32 (D), its sum over
 * tokens (must be NULL iff delta_bias is NULL; deterministic). The forward and
 * backward must be given the same options. selective_scan_pack_fwd and
 * selective_scan_pack_bwd are these with (NULL, 0, 0.0f).
 * Errors as selective_scan_pack_fwd / _bwd.
 */
int selective_scan_pack_fwd_ex(const void *u, const void *delta, const float *A, const void *B,
                               const void *C, const float *Dskip, const void *z, const int32_t *pos,
                               void *out, void *workspace, size_t workspace_bytes,
                               int64_t T, int32_t D, int32_t N, int32_t dtype,
                               const float *delta_bias, int32_t delta_softplus, float gate_floor,
                               void *stream);
int selective_scan_pack_bwd_ex(const void *u, const void *delta, const float *A, const void *B,
                               const void *C, const float *Dskip, const void *z, const int32_t *pos,
                               const void *dout, void *workspace, size_t workspace_bytes,
                               void *du, void *ddelta, float *dA, float *dB, float *dC,
                               float *dD, void *dz,
                               int64_t T, int32_t D, int32_t N, int32_t dtype,
                               const float *delta_bias, int32_t delta_softplus, float gate_floor,
                               float *ddelta_bias, void *stream);

/*
 * selective_scan_pack_fwd_states / _bwd_states — sequences that start from a
 * given state and hand on their last one.
 * [P5] section "结论与讨论" proposes cutting a sequence that overruns a pack into
 * pieces that keep passing state, so packs need no padding; [P1] section 3.2
 * runs long documents segment by segment, resetting or passing the SSM state
 * at segment starts. These are the _ex entry points plus, per sequence s of
 * cu_seqlens (device int32 [nseq+1], the one pos was built from):
 *   initial_state   fp32 (nseq, D, N), nullable (zero): the state before the
 *                   sequence's first token, h_{-1} = initial_state[s]; the
 *                   recurrence then runs unchanged
 *   final_state     fp32 (nseq, D, N) out, nullable: the state after its last
 *                   token (initial_state[s], or zero, for an empty sequence)
 *   dfinal_state    fp32 (nseq, D, N), nullable (zero): dL/d final_state
 *   dinitial_state  fp32 (nseq, D, N) out, nullable: dL/d initial_state
 * Element (s, d, n) is at (s*D + d)*N + n. A piece that continues a sequence
 * gets the previous piece's final_state as its initial_state, and the
 * previous piece's backward gets this piece's dinitial_state as its
 * dfinal_state (so the later pack's backward runs first). The backward must
 * be given the forward's initial_state. With every state pointer NULL these
 * are the _ex entry points (cu_seqlens and nseq are then not read).
 * Errors as the _ex entry points, plus SSMP_ERR_NULL (a state pointer without
 * cu_seqlens) and SSMP_ERR_SHAPE (nseq < 1 with a state pointer).
 */
int selective_scan_pack_fwd_states(const void *u, const void *delta, const float *A, const void *B,
                                   const void *C, const float *Dskip, const void *z, const int32_t *pos,
                                   void *out, void *workspace, size_t workspace_bytes,
                                   int64_t T, int32_t D, int32_t N, int32_t dtype,
                                   const float *delta_bias, int32_t delta_softplus, float gate_floor,
                                   const int32_t *cu_seqlens, int32_t nseq,
                                   const float *initial_state, float *final_state, void *stream);
int selective_scan_pack_bwd_states(const void *u, const void *delta, const float *A, const void *B,
                                   const void *C, const float *Dskip, const void *z, const int32_t *pos,
                                   const void *dout, void *workspace, size_t workspace_bytes,
                                   void *du, void *ddelta, float *dA, float *dB, float *dC,
                                   float *dD, void *dz,
                                   int64_t T, int32_t D, int32_t N, int32_t dtype,
                                   const float *delta_bias, int32_t delta_softplus, float gate_floor,
                                   float *ddelta_bias, const int32_t *cu_seqlens, int32_t nseq,
                                   const float *initial_state, const float *dfinal_state,
                                   float *dinitial_state, void *stream);

/*
 * selective_scan_pack_fwd_ck / _bwd_ck — the _states entry points with the
 * memory kept between forward and backward chosen by the caller. The
 * recurrence of [P5] "SSM_pack算子" is sequential in t, so the backward,
 * which walks t in reverse, restarts from states the forward kept. The
 * single workspace of the other entry points is split in two:
 *   saved    kept by the caller from the forward to the backward (the only
 *            per-layer memory between them): fp32 states entering every
 *            ckpt_interval-th token, selective_scan_pack_saved_bytes(T, D,
 *            N, ckpt_interval) bytes. Written by the forward, read by the
 *            backward, which must get the same inputs and options.
 *   scratch  used during one call only and free again when the call's work
 *            on `stream` is done: selective_scan_pack_fwd_scratch_bytes(T,
 *            D, N) for the forward, selective_scan_pack_bwd_scratch_bytes(T,
 *            D, N, ckpt_interval) for the backward.
 * ckpt_interval is 0 or a power of two from 4 to 2048:
 *   4, 8     the backward reads the kept states directly (fastest backward;
 *            the _states entry points use 8, their workspace being saved
 *            followed by scratch);
 *   16..2048 fewer kept states; the backward first replays the forward's
 *            recurrence from them into states 8 tokens apart in its scratch;
 *   0        nothing kept (saved may be NULL; a forward-only call, e.g. for
 *            inference); a backward then recomputes every state from the
 *            inputs.
 * The forward's outputs do not depend on ckpt_interval. The backward's
 * replay repeats the forward's arithmetic within each forward chunk (64 or
 * more tokens), so intervals 0 to 64 give the interval-8 gradients bit for
 * bit; a longer interval replays across chunk boundaries where the forward
 * restarted from its chunk carry, which changes gradients by rounding only.
 * Other arguments, outputs and
 * errors as the _states entry points; ckpt_interval outside the set above
 * is SSMP_ERR_SHAPE, a missing or short saved or scratch buffer
 * SSMP_ERR_WORKSPACE. The size queries return 0 for arguments out of range.
 */
size_t selective_scan_pack_saved_bytes(int64_t T, int32_t D, int32_t N, int32_t ckpt_interval);
size_t selective_scan_pack_fwd_scratch_bytes(int64_t T, int32_t D, int32_t N);
size_t selective_scan_pack_bwd_scratch_bytes(int64_t T, int32_t D, int32_t N, int32_t ckpt_interval);
int selective_scan_pack_fwd_ck(const void *u, const void *delta, const float *A, const void *B,
                               const void *C, const float *Dskip, const void *z, const int32_t *pos,
                               void *out, int64_t T, int32_t D, int32_t N, int32_t dtype,
                               const float *delta_bias, int32_t delta_softplus, float gate_floor,
                               const int32_t *cu_seqlens, int32_t nseq,
                               const float *initial_state, float *final_state,
                               int32_t ckpt_interval, void *saved, size_t saved_bytes,
                               void *scratch, size_t scratch_bytes, void *stream);
int selective_scan_pack_bwd_ck(const void *u, const void *delta, const float *A, const void *B,
                               const void *C, const float *Dskip, const void *z, const int32_t *pos,
                               const void *dout, void *du, void *ddelta, float *dA, float *dB,
                               float *dC, float *dD, void *dz,
                               int64_t T, int32_t D, int32_t N, int32_t dtype,
                               const float *delta_bias, int32_t delta_softplus, float gate_floor,
                               float *ddelta_bias, const int32_t *cu_seqlens, int32_t nseq,
                               const float *initial_state, const float *dfinal_state,
                               float *dinitial_state, int32_t ckpt_interval, const void *saved,
                               size_t saved_bytes, void *scratch, size_t scratch_bytes,
                               void *stream);

/*
 * selective_scan_pack_fwd_noalloc — selective_scan_pack_fwd_ck with
 * ckpt_interval 0 (forward only, nothing kept) that allocates nothing and
 * takes no workspace. For callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid it.
 * Its scratch is a buffer of SSMP_NOALLOC_SCRATCH_BYTES inside the library,
 * one per device, held by every device the library runs on until the
 * process ends; a problem whose selective_scan_pack_fwd_scratch_bytes
 * exceeds it is refused with SSMP_ERR_TOO_LARGE (with d_state 16: beyond
 * about 256k tokens at d_inner 1536, 342k at 4096, 112k at 16384). Every
 * call on a device shares that device's
 * buffer: calls that may overlap on one device (different streams, or
 * several host threads) race and must be serialised by the caller; calls in
 * order on one stream are safe. The buffer needs no clearing between calls.
 * The caller still passes inputs and outputs; other arguments, results and
 * errors as selective_scan_pack_fwd_ck.
 */
#define SSMP_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int selective_scan_pack_fwd_noalloc(const void *u, const void *delta, const float *A, const void *B,
                                    const void *C, const float *Dskip, const void *z,
                                    const int32_t *pos, void *out, int64_t T, int32_t D, int32_t N,
                                    int32_t dtype, const float *delta_bias, int32_t delta_softplus,
                                    float gate_floor, const int32_t *cu_seqlens, int32_t nseq,
                                    const float *initial_state, float *final_state, void *stream);

/* Packing strategies of varlen_pack_plan. */
enum ssmp_pack_strategy {
    SSMP_PACK_SEQUENTIAL = 0,   /* arrival order, seal when the next does not fit */
    SSMP_PACK_LOCAL_GREEDY = 1  /* first-fit decreasing inside windows */
};

/*
 * varlen_pack_plan — which sequences share a pack of `capacity` tokens.
 * [P5] section "结论与讨论": the article packs sequences in arrival order,
 * sealing a pack when the next sequence does not fit (19.1% padding on its
 * pretraining corpus), and notes that sorting a window of pending sequences
 * and packing them greedily brings padding down to as little as 0.46%.
 * SSMP_PACK_LOCAL_GREEDY takes the greedy rule to be first-fit decreasing
 * inside each run of `window` consecutive sequences: longest first, ties in
 * arrival order, each into the lowest-numbered pack of the window with room,
 * the window's packs sealed when it ends. Deterministic.
 *
 * HOST function: every pointer is a host pointer; the call is synchronous,
 * uses no GPU and allocates only host scratch (O(window)).
 *   lengths      int32 [nseq], 0 <= lengths[i] <= capacity, arrival order
 *   window       sequences per window (LOCAL_GREEDY; >= 1); ignored otherwise
 *   order        int32 [nseq] out: sequence indices, pack by pack
 *   pack_bounds  int32 [nseq+1] out: pack p holds order[pack_bounds[p] ..
 *                pack_bounds[p+1]); entries 0..n_packs are written
 *   cu_seqlens   int32 [nseq+1] out: cumulative lengths along `order`, the
 *                cu_seqlens of the packed batch without padding tokens
 *   max_seqlen   int32 [nseq] out: longest sequence of each pack (0..n_packs-1)
 *   n_packs      int32 [1] out
 *   padding      int64 [1] out: n_packs * capacity - sum(lengths)
 * Errors: SSMP_ERR_NULL, SSMP_ERR_SHAPE (nseq < 0, capacity < 1, a length
 * outside [0, capacity], window < 1 for LOCAL_GREEDY, total >= 2^31),
 * SSMP_ERR_UNSUPPORTED (unknown strategy). Arguments are checked before
 * any output is written.
 */
int varlen_pack_plan(const int32_t *lengths, int32_t nseq, int32_t capacity, int32_t strategy,
                     int32_t window, int32_t *order, int32_t *pack_bounds, int32_t *cu_seqlens,
                     int32_t *max_seqlen, int32_t *n_packs, int64_t *padding);

#ifdef __cplusplus
}
#endif

#endif /* SSMPACK_H */
