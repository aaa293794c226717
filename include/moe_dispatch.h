/*
 * moe_dispatch.h -- C ABI of the single-layer MoE training hot path for AMD
 * MI355X (gfx950): atomic-free construction of the routing index structures,
 * the gather-on-the-fly expert FFN forward, and its backward.
 *
 * The operations follow the MoEBlaze wiki note ("MoEBlaze: Breaking the
 * Memory Wall for Efficient MoE Training on Modern GPUs", awesome-system-papers
 * wiki), section "Core method":
 *   - sub-section "materialisation-free token dispatch": the four index
 *     structures (data-structure table) and the forward/backward that gather
 *     from and scatter into the original (L, d) tensors through them;
 *   - sub-section "atomic-free three-step dispatch construction": token-expert
 *     map, per-expert length count with prefix sum, tile scan and scatter;
 *   - sub-section "SwiGLU kernel fusion + activation checkpoint": one load of
 *     x for both first-layer projections, activation in the epilogue, only the
 *     first-MLP outputs A and B kept for backward, SiLU recomputed there.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers on the calling thread's current
 *     HIP device, row-major and contiguous.  The caller owns every buffer; the
 *     library never allocates, frees or synchronises.  All work is enqueued on
 *     `stream` (a hipStream_t; NULL = the null stream) and the call returns
 *     before it runs.  A call launches kernels only (no copy, no memset; no
 *     event either while the kernel timers of moe_profile_enable are off, the
 *     default), so a sequence of calls can be captured into a HIP graph on a
 *     capturing stream and replayed; the graph keeps the pointers it was
 *     captured with.
 *   - Workspace: pass ws == NULL to query; the required size is written to
 *     *ws_bytes, MOE_OK is returned and nothing is launched.  Otherwise
 *     *ws_bytes is the size of `ws` (device memory, 256-byte aligned); if it is
 *     too small the call returns MOE_ERR_WORKSPACE.  Workspace contents need
 *     no initialisation and are not meaningful after the call.
 *   - Arguments are validated on the host before any HIP call.  A call that
 *     returns anything but MOE_OK has launched nothing and written nothing.
 *     moe_last_error() then describes the problem (thread-local text).
 *   - HIP launch errors are returned as MOE_ERR_HIP.
 *   - Limits: 1 <= L; 1 <= E <= 1024; 1 <= K <= min(E, 255), and K <= 8 when
 *     E > 256; L*K < 2^31.
 *     FFN calls also need d % 8 == 0 and h % 8 == 0, d and h at most
 *     MOE_MAX_WIDTH (in-tile byte offsets of the GEMM epilogues are 32-bit),
 *     and every x, W, A, B, y, dy, dx, dW pointer 16-byte aligned.  Integer
 *     and float32 index/gate arrays must be 4-byte aligned.  Shapes outside
 *     these limits return MOE_ERR_UNSUPPORTED.
 *   - Router logits must be finite; NaN or infinite logits give unspecified
 *     (but memory-safe) results: the gates are unspecified, yet every token
 *     still receives K distinct experts, so the four index structures keep
 *     their layout and stay valid inputs of the FFN calls.
 *   - Results are deterministic: repeated calls on the same inputs produce
 *     bitwise-identical outputs.
 */
#ifndef MOE_DISPATCH_H
#define MOE_DISPATCH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null pointer, bad size, bad enum value        */
  MOE_ERR_UNSUPPORTED = 2, /* valid request outside the limits above        */
  MOE_ERR_WORKSPACE = 3,   /* *ws_bytes smaller than the queried size       */
  MOE_ERR_HIP = 4          /* a HIP runtime call or launch failed           */
};

/* Largest model width d and expert hidden width h the FFN calls accept. */
#define MOE_MAX_WIDTH 1048576

/* Element type of x, W1, W3, W2, A, B, y, dy, dx, dW1, dW3, dW2.
 * Router logits and gates are always float32; accumulation is float32. */
enum { MOE_F32 = 0, MOE_BF16 = 1 };

/* Expert FFN kind.
 *   MOE_SILU:   FFN_e(x) = SiLU(x W1_e) W2_e
 *   MOE_SWIGLU: FFN_e(x) = (SiLU(x W1_e) * (x W3_e)) W2_e
 * (W1 = gate projection, W3 = up projection, W2 = down projection.) */
enum { MOE_SILU = 0, MOE_SWIGLU = 1 };

/* Flags of moe_shape.flags (0 = none).
 *   MOE_FLAG_RECOMPUTE_G: keep no [L*K, h] copy of G = SiLU(A) [* B]
 *     between the two GEMMs of either pass.  The forward stores only A and
 *     B; before each of its K slot passes it forms that pass's L rows of G
 *     from A and B into an [L, h] piece of the workspace, and the backward
 *     forms gate * G the same way for dW2, one group of experts (at most L
 *     routes) at a time, before dA, dB replace A, B.  The workspace then
 *     holds one [L, h] piece instead of the [L*K, h] buffer, at the price
 *     of reading A and B once more per piece.  Results agree with the
 *     default within the bf16 rounding of G (G is formed from the stored
 *     A, B instead of their float32 accumulators). */
enum { MOE_FLAG_RECOMPUTE_G = 1 };

typedef struct moe_shape {
  int64_t L;     /* tokens                                  */
  int32_t d;     /* model width                             */
  int32_t h;     /* expert hidden width                     */
  int32_t E;     /* experts                                 */
  int32_t K;     /* experts per token (top-K)               */
  int32_t dtype; /* MOE_F32 or MOE_BF16                     */
  int32_t act;   /* MOE_SILU or MOE_SWIGLU                  */
  int32_t flags; /* MOE_FLAG_* bits, 0 for none (FFN calls)  */
} moe_shape;

/*
 * moe_dispatch_build -- routing and the four index structures.
 *
 * Passage: wiki note, "Core method" > "materialisation-free token dispatch"
 * (data-structure table) and "atomic-free three-step dispatch construction".
 * Uses s->L, s->E, s->K only.
 *
 * In:  logits  [L, E] float32, router logits.
 * Out: token_expert_indices [L, K] int32: each token's K experts, the K largest
 *        logits with ties at the K-th place going to the lower expert id,
 *        listed in ascending expert id ("slot" k = position in this list).
 *      gates [L, K] float32: softmax over the token's K selected logits, in
 *        slot order.
 *      expert_token_offsets [E + 1] int32: offsets[0] = 0, offsets[E] = L*K;
 *        expert e owns rows [offsets[e], offsets[e+1]).
 *      expert_token_indices [L*K] int32: for each expert in ascending order,
 *        its tokens in ascending order.
 *      token_index_map [L, K] int32: absolute row p of token t's slot-k route
 *        in expert_token_indices (expert_token_indices[p] == t).
 * Row p of the FFN's A and B buffers is route p.
 * The build writes every output element exactly once and uses no atomics.
 */
int moe_dispatch_build(const moe_shape* s, const float* logits,
                       int32_t* expert_token_indices, int32_t* expert_token_offsets,
                       int32_t* token_expert_indices, int32_t* token_index_map,
                       float* gates, void* ws, size_t* ws_bytes, void* stream);

/*
 * moe_dispatch_build_noalloc -- moe_dispatch_build without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).
 *
 * Same inputs, outputs, validation and results as moe_dispatch_build.  The
 * workspace is a device array owned by the library, MOE_NOALLOC_WS_BYTES
 * bytes per GPU, held from the first call on that GPU until the process
 * ends; the call itself allocates nothing.  A shape whose moe_dispatch_build
 * workspace exceeds MOE_NOALLOC_WS_BYTES returns MOE_ERR_UNSUPPORTED (the
 * layer with L = 1,048,576 tokens, E = 64, K = 6 needs 21 MiB and fits).
 * Every call on one GPU uses the same array: calls that can overlap in time
 * on one GPU (unordered streams, several host threads) race and give
 * undefined results; calls ordered on one stream are safe.
 */
#define MOE_NOALLOC_WS_BYTES (24u << 20)
int moe_dispatch_build_noalloc(const moe_shape* s, const float* logits,
                               int32_t* expert_token_indices, int32_t* expert_token_offsets,
                               int32_t* token_expert_indices, int32_t* token_index_map,
                               float* gates, void* stream);

/*
 * moe_ffn_forward -- expert FFN forward with on-the-fly gather and
 * gate-weighted aggregation.
 *
 * Passage: wiki note, "Core method" > "materialisation-free token dispatch"
 * (forward paragraph) and "SwiGLU kernel fusion + activation checkpoint".
 *
 * For route p (expert e, token t = expert_token_indices[p]):
 *   A[p] = x[t] W1_e,  B[p] = x[t] W3_e (SwiGLU),  G = SiLU(A) [* B],
 *   O[p] = G W2_e,   y[t] = sum over slots k (ascending) of gates[t,k] * O[p(t,k)].
 * Rows of x are gathered through expert_token_indices; no (L*K, d) buffer
 * is formed.  The sum over k is taken in ascending slot order in float32.
 *
 * In:  x [L, d]; W1 [E, d, h]; W3 [E, d, h] (SwiGLU; ignored for SiLU);
 *      W2 [E, h, d]; the index structures and gates from moe_dispatch_build.
 * Out: y [L, d]; A [L*K, h]; B [L*K, h] (SwiGLU; ignored for SiLU).
 *      A and B are the activation checkpoint consumed by moe_ffn_backward.
 */
int moe_ffn_forward(const moe_shape* s, const void* x, const void* W1, const void* W3,
                    const void* W2, const int32_t* expert_token_indices,
                    const int32_t* expert_token_offsets, const int32_t* token_expert_indices,
                    const int32_t* token_index_map, const float* gates, void* y, void* A,
                    void* B, void* ws, size_t* ws_bytes, void* stream);

/*
 * moe_ffn_backward -- gradients of the layer for dx, dW1, dW3, dW2.
 *
 * Passage: wiki note, "Core method" > "materialisation-free token dispatch"
 * (backward paragraph) and the activation-checkpoint paragraph of "SwiGLU
 * kernel fusion + activation checkpoint".
 *
 * dy is scattered to routes through the same index structures
 * (dO[p] = gates[t,k] * dy[t]); SiLU(A) is recomputed from the checkpoint:
 *   dW2_e = G^T dO,  dG = dO W2_e^T,
 *   SwiGLU: dA = dG * B * SiLU'(A), dB = dG * SiLU(A);  SiLU: dA = dG * SiLU'(A),
 *   dW1_e = X^T dA,  dW3_e = X^T dB,
 *   dx[t] = sum over slots k (ascending) of (dA W1_e^T + dB W3_e^T)[p(t,k)].
 *
 * In:  dy [L, d], x, W1, W3, W2, index structures and gates as in forward;
 *      A, B: the checkpoint written by moe_ffn_forward for the same inputs.
 * Out: dx [L, d]; dW1, dW3 [E, d, h]; dW2 [E, h, d].  dW outputs are
 *      overwritten (not accumulated); an expert with no routes gets exact 0.
 *      dlogits [L, E] float32, optional (NULL: not computed): the gradient
 *      with respect to the router logits.  The pages do not describe it; it
 *      is the derivative of the same forward with the gates a softmax over
 *      the K selected logits:
 *        dg[t,k] = <dy[t], O[p(t,k)]>  (O = the route's un-gated output G W2_e),
 *        dlogits[t, e_k] = gates[t,k] * (dg[t,k] - sum_j gates[t,j] dg[t,j]),
 *      0 for the experts a token did not select (the selection is piecewise
 *      constant).  dg is formed in float32 from the recomputed G and
 *      dy W2_e^T, summed over 256-column tiles in a fixed order.
 * Clobbers A and B (they hold dA and dB on return).
 */
int moe_ffn_backward(const moe_shape* s, const void* dy, const void* x, const void* W1,
                     const void* W3, const void* W2, const int32_t* expert_token_indices,
                     const int32_t* expert_token_offsets, const int32_t* token_expert_indices,
                     const int32_t* token_index_map, const float* gates, void* A, void* B,
                     void* dx, void* dW1, void* dW3, void* dW2, float* dlogits, void* ws,
                     size_t* ws_bytes, void* stream);

/* Text describing the last non-OK return on the calling thread ("" if none).
 * The pointer stays valid until the next call on the same thread. */
const char* moe_last_error(void);

/*
 * Kernel timing (instrumentation for measurement, not part of the layer's
 * arithmetic).  While enabled, each kernel launch of the three calls above is
 * bracketed by a pair of HIP events recorded on the same stream.
 * moe_profile_read() waits for those events, adds each kernel's elapsed time
 * to per-kernel totals and returns them; moe_profile_reset() clears totals.
 * Not thread-safe: enable it from one host thread.
 */
typedef struct moe_kernel_stat {
  char name[32];     /* kernel name                          */
  int64_t launches;  /* launches timed                       */
  double total_ms;   /* summed event-to-event time           */
} moe_kernel_stat;

int moe_profile_enable(int on);
int moe_profile_reset(void);
/* Writes up to max_stats entries, sets *n_stats to the number of kernels. */
int moe_profile_read(moe_kernel_stat* stats, int max_stats, int* n_stats);

#ifdef __cplusplus
}
#endif

#endif /* MOE_DISPATCH_H */
