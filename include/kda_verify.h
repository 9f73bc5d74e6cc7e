/*
 * kda_verify.h - C ABI of the MI355X (gfx950) fused causal-conv1d + Kimi Delta
 * Attention (KDA) multi-token verify-decode step.
 *
 * The operation is the one described on the cuLA pull request page "[KDA] Fuse
 * causal conv1d into MTP verify decode #107" (PR description): a width-4 depthwise
 * causal conv1d with SiLU over packed pre-convolution q/k/v activations, q/k L2
 * normalisation, a per-channel decay gate (softplus or safe form) and a sigmoid
 * beta, then the gated delta rule over T draft tokens with verify semantics:
 *
 *   S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *   o_t = S_t^T q_t,
 *
 * the persistent state S_{-1} is only read; each S_t goes to inter_ssm, each o_t to o;
 * each token's raw conv window goes to conv_window, and conv_state is rolled in place
 * to the last three raw tokens.
 *
 * Conventions for every entry point:
 *   - Pointers are device pointers (hipMalloc'd or from a caching allocator) unless
 *     said otherwise. The caller owns every buffer it passes; the library keeps no
 *     pointer to them after a call returns and allocates no device memory (the
 *     counters of kda_conv_verify_decode_noalloc are a static array that is loaded
 *     with the library).
 *   - Arrays are dense, row-major and contiguous. Every device base pointer must be
 *     16-byte aligned (KDA_ERR_ALIGN otherwise).
 *   - Calls are asynchronous on `stream` (NULL = the default stream); none blocks the
 *     host. A call that returns an error launched nothing and wrote nothing.
 *   - No entry point throws; errors are returned as kda_status.
 */
#ifndef KDA_VERIFY_H
#define KDA_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KDA_OK = 0,
  KDA_ERR_NULL = -1,        /* a required pointer is NULL */
  KDA_ERR_SHAPE = -2,       /* a size is out of range or inconsistent (e.g. HV % H != 0) */
  KDA_ERR_UNSUPPORTED = -3, /* valid but not built: (K, V) pair, dtype, gate or variant */
  KDA_ERR_ALIGN = -4,       /* a device pointer is not 16-byte aligned */
  KDA_ERR_WORKSPACE = -5,   /* workspace missing or smaller than kda_workspace_bytes() */
  KDA_ERR_LAUNCH = -6,      /* the HIP runtime reported an error at launch */
  KDA_ERR_ALIAS = -7,       /* a written buffer overlaps another buffer */
  KDA_ERR_SCRATCH = -8      /* kda_conv_verify_decode_noalloc: the shape needs more counter
                               words than its static scratch holds */
} kda_status;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

/* Gate forms (PR#107 description: softplus gate and safe gate with a lower bound).
 * With gamma = gate + dt_bias:
 *   KDA_GATE_SOFTPLUS: log alpha = -exp(A_log) * softplus(gamma), where
 *       softplus(x) = log(1 + exp(b x)) / b if b x <= threshold, else x
 *       (a true branch; the exponential is never formed past the threshold,
 *        PR#107 code review);
 *   KDA_GATE_SAFE:     log alpha = lower_bound * sigmoid(exp(A_log) * gamma). */
typedef enum { KDA_GATE_SOFTPLUS = 0, KDA_GATE_SAFE = 1 } kda_gate_mode;

/* Kernel variant (PR#107 description: two variants, one API and one arithmetic).
 * AUTO picks from N*HV and T; SMALL splits each value head's V columns over several
 * workgroups; LARGE gives each (sequence, value head) one workgroup. Both variants
 * return bit-identical results. */
typedef enum { KDA_VARIANT_AUTO = 0, KDA_VARIANT_SMALL = 1, KDA_VARIANT_LARGE = 2 } kda_variant;

typedef struct {
  int32_t N;  /* sequences, >= 0 (N = 0 is a no-op) */
  int32_t T;  /* draft tokens per sequence, 1 <= T <= KDA_MAX_T (any T >= 1, PR#107 commit 1) */
  int32_t H;  /* q/k heads, >= 1 */
  int32_t HV; /* value heads, a multiple of H; value head hv reads q/k head hv / (HV/H) */
  int32_t K;  /* q/k head dim; (K, V) in {(16,16), (64,64), (128,128)} */
  int32_t V;  /* value head dim */
  int32_t in_dtype;  /* kda_dtype of mixed_qkv, conv_weight, conv_state, conv_window, gate, beta, o */
  int32_t gate_mode; /* kda_gate_mode */
  int32_t variant;   /* kda_variant */
  float lower_bound;        /* safe gate bound, default -5.0 */
  float softplus_beta;      /* default 1.0, must be > 0 */
  float softplus_threshold; /* default 20.0 */
  float scale;              /* q scale; <= 0 selects K^-1/2 */
  float l2norm_eps;         /* q/k l2norm: x / sqrt(sum x^2 + eps); default 1e-6, >= 0 */
  /* Tuning overrides (0 = chosen from the shape). They change speed only, never results:
   * every tile width and store policy gives the same bits. */
  int32_t tile_columns;     /* V columns per workgroup: 32, 64 or 128 (K = V = 128 only);
                               V selects LARGE, fewer SMALL, and overrides `variant` */
  int32_t store_policy;     /* snapshot stores: 1 streaming (non-temporal hint), 2 streaming
                               at device scope (non-temporal hint with device coherence) */
  int32_t max_wg_per_cu;    /* at most 1, 2, 4 or 6 workgroups per compute unit, by reserving
                               LDS per workgroup (fewer concurrent snapshot streams can use
                               HBM better); the kernel's own limits still apply. 8: no cap.
                               0: the AUTO cap with the AUTO tile, none when tile_columns or
                               `variant` picks the tile */
  int32_t column_groups;    /* 1, 2 or 4: a whole-V workgroup (K = V = 128) runs as that many
                               groups of 4 wave64s over 128/groups columns each, sharing the
                               staged inputs and the conv (not for fp32 inputs at T > 8).
                               0: the AUTO choice with the AUTO tile, 1 with a caller's tile */
  int32_t schedule;         /* 1 grid: one workgroup per unit, started by the hardware as
                               slots free up; 2 queue: only as many workgroups as are
                               resident at once (compute units x max_wg_per_cu, or the
                               kernel's occupancy without a cap), each pulling units from
                               a counter in the workspace until none are left. The queue
                               needs whole-V workgroups (with K = V = 128: tile 128, not
                               fp32 inputs at T > 8; with K = V = 64: not the SMALL
                               variant) and the fused step (the unfused form rejects it).
                               3 stream: the queue with a fifth wave per workgroup that
                               loads each unit's inputs and state tile into LDS while the
                               other four compute the unit before it; K = V = 128, whole-V
                               workgroups of one column group, one per compute unit, T <= 8,
                               the fused step.
                               0: the AUTO choice with the AUTO tile, the grid with a
                               caller's tile */
  int32_t unit_order;       /* grid schedule only: the order in which units are dealt to
                               the 8 XCDs (workgroups go to them round-robin). 1 XCD ranges:
                               each XCD takes one contiguous range of units; 2 pairs: pairs
                               of neighbouring units go to the XCDs in turn. 0: pairs when
                               whole-V workgroups run without a cap (all resident at once),
                               XCD ranges otherwise */
  int32_t prefetch;         /* stream schedule only (ignored otherwise): when a workgroup
                               loads its next unit's state tile. 1 once the current unit's
                               conv phase is done; 2 as soon as the compute waves hold the
                               current unit's state in registers. 0: 2 up to 65536
                               snapshot tiles (N * HV * T) per call, 1 beyond */
} kda_verify_params;

#define KDA_MAX_T 16

/* Fill *p with the shape and the defaults above (AUTO variant, softplus gate, bf16). */
void kda_verify_params_init(kda_verify_params* p, int32_t N, int32_t T, int32_t H, int32_t HV,
                            int32_t K, int32_t V);

/* Bytes of device workspace kda_conv_verify_decode needs for these params (one
 * uint32 arrival counter per (sequence, q/k head), then the queue schedule's two
 * counters: units handed out and workgroups done; rounded up to 256). The arrival
 * counters decide which workgroup writes the q/k part of conv_state, which several
 * workgroups read (PR#107 description: last-arrival counters). All of them must be
 * zero before the first call (kda_workspace_reset); each call leaves them zero again.
 * Returns 0 for invalid params. */
size_t kda_workspace_bytes(const kda_verify_params* p);

/* Zero `bytes` of workspace on `stream` with a fill kernel (graph-capturable). Use it
 * once after allocation, and after a call that did not run to completion (PR#107 code
 * review: stale counters would corrupt later calls). */
kda_status kda_workspace_reset(void* workspace, size_t bytes, hipStream_t stream);

/* The variant AUTO resolves to for these params (host-only, no HIP call), or a
 * negative kda_status for invalid params. */
int32_t kda_select_variant(const kda_verify_params* p);

/* The launch configuration kda_conv_verify_decode would use for these params (after the
 * overrides): V columns per workgroup, snapshot store policy (1 streaming, 2 streaming at
 * device scope), workgroups-per-CU cap (0 = none), column groups per workgroup, schedule
 * (1 grid, 2 queue, 3 stream), unit order (1 XCD ranges, 2 pairs; the queue and the
 * stream take their first round in XCD ranges) and the stream's state prefetch (1, 2;
 * 0 for the other schedules). Host-only; any output pointer may be NULL. Returns the
 * params' validation status (outputs untouched unless KDA_OK). */
kda_status kda_select_launch(const kda_verify_params* p, int32_t* tile_columns, int32_t* store_policy,
                             int32_t* max_wg_per_cu, int32_t* column_groups, int32_t* schedule,
                             int32_t* unit_order, int32_t* prefetch);

/* Validate params and pointers without launching (host-only, no HIP call). */
kda_status kda_validate(const kda_verify_params* p, const void* mixed_qkv, const void* conv_weight,
                        const void* conv_state, const void* gate, const float* A_log,
                        const float* dt_bias, const void* beta, const float* state, const void* o,
                        const float* inter_ssm, const void* conv_window, const void* workspace,
                        size_t workspace_bytes);

/* One fused verify step (PR#107 description). C = 2*H*K + HV*V.
 *   mixed_qkv   [N,T,C]      in_dtype, read.  Channels q (H*K) | k (H*K) | v (HV*V), head-major.
 *   conv_weight [C,4]        in_dtype, read.  Tap 3 multiplies the newest token; no bias.
 *   conv_state  [N,C,3]      in_dtype, read, then overwritten in place with the last three raw
 *                            tokens of the extended sequence (old cache, then the T new tokens).
 *   gate        [N,T,HV,K]   in_dtype, read.  Raw gate input.
 *   A_log       [HV]         fp32, read.
 *   dt_bias     [HV*K]       fp32, read.
 *   beta        [N,T,HV]     in_dtype, read.  beta_t = sigmoid(beta).
 *   state       [N,HV,K,V]   fp32, read only. Must not overlap inter_ssm.
 *   o           [N,T,HV,V]   in_dtype, written (rounded to nearest even from fp32).
 *   inter_ssm   [N,T,HV,K,V] fp32, written: the state after each token.
 *   conv_window [N,T,C,3]    in_dtype, written: conv_window[n,t,c,:] is the conv cache to
 *                            restore if tokens 0..t are accepted (bit copies of raw inputs).
 *   workspace   >= kda_workspace_bytes(p) bytes, zeroed before first use; calls that
 *               run at the same time need separate workspaces.
 * q and k are L2-normalised per head after conv + SiLU, q is multiplied by `scale`;
 * v is not normalised. Arithmetic is fp32; conv_window and conv_state are exact copies. */
kda_status kda_conv_verify_decode(const kda_verify_params* p, const void* mixed_qkv,
                                  const void* conv_weight, void* conv_state, const void* gate,
                                  const float* A_log, const float* dt_bias, const void* beta,
                                  const float* state, void* o, float* inter_ssm, void* conv_window,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Pool indirection (PR#107 PR description: conv_state_indices, cache_indices and
 * intermediate_state_indices, each normalised on its own). Each array is a device
 * int32 array of N entries, or NULL for the identity (sequence n uses row n, and the
 * pool then has N rows). Sequence n is a padding entry when any of its three indices is
 * negative or not below the pool's row count: nothing is read or written for it (its
 * rows of o are left as they were). Rows written by one verify call (conv_state and the
 * two intermediate pools) must be distinct across the batch; a verify call only reads the
 * state pool, so sequences may share a state row there (a commit writes it: see
 * kda_verify_commit). The library does not read the device index arrays on the host, so
 * it cannot check distinctness: duplicated written rows race, and such a row ends up
 * holding an unspecified mix of the sequences' values.
 * When every sequence of a batch advances every step, a call's snapshots can serve as the
 * next call's pools, with no accept step in between: inter_ssm [P,T,HV,K,V] is also a
 * state pool of P*T rows [HV,K,V], and conv_window [P,T,C,3] a conv_state pool of P*T
 * rows [C,3], so cache_indices[n] = conv_state_indices[n] = r*T + a - 1 (r the sequence's
 * intermediate row in the previous call, a its accepted tokens) starts sequence n from the
 * accepted token's state and conv window. That call writes its own snapshots to a second
 * pair of buffers (the two pairs alternate), and rolls the conv cache into the old
 * conv_window row it read. The results are the bits of verify -> kda_verify_commit. */
typedef struct {
  const int32_t* conv_state_indices;         /* row of conv_state [conv_state_slots, C, 3] */
  const int32_t* cache_indices;              /* row of state [state_slots, HV, K, V] */
  const int32_t* intermediate_state_indices; /* row of inter_ssm [intermediate_slots, T, HV, K, V]
                                                and conv_window [intermediate_slots, T, C, 3] */
  int32_t conv_state_slots;
  int32_t state_slots;
  int32_t intermediate_slots;
} kda_pool_desc;

/* kda_conv_verify_decode on pooled buffers: conv_state, state, inter_ssm and conv_window
 * are the pools described by *pools (row counts instead of N); mixed_qkv, gate, beta and o
 * keep their per-call [N, ...] shapes. pools == NULL is the identity (the same as
 * kda_conv_verify_decode). Same validation and error behaviour. */
kda_status kda_conv_verify_decode_pooled(const kda_verify_params* p, const kda_pool_desc* pools,
                                         const void* mixed_qkv, const void* conv_weight,
                                         void* conv_state, const void* gate, const float* A_log,
                                         const float* dt_bias, const void* beta, const float* state,
                                         void* o, float* inter_ssm, void* conv_window,
                                         void* workspace, size_t workspace_bytes,
                                         hipStream_t stream);

/* The same step in unfused form, for measuring what fusion saves (PR#107 PR description:
 * fusing removes a separate conv launch and intermediate HBM round trips). A first kernel
 * runs the conv + SiLU over all channels and writes the activations to act [N,T,C]
 * (fp32), the conv windows and the rolled cache; a second kernel runs the rest of the
 * step from act. Same arguments, pools and validation as kda_conv_verify_decode_pooled,
 * plus act (device, 16-byte aligned, not overlapping any other buffer). The activations
 * stay fp32 so that the results keep the fused step's accuracy (rounding them to bf16
 * moves inter_ssm by up to ~6e-3). */
kda_status kda_conv_verify_decode_unfused(const kda_verify_params* p, const kda_pool_desc* pools,
                                          const void* mixed_qkv, const void* conv_weight,
                                          void* conv_state, const void* gate, const float* A_log,
                                          const float* dt_bias, const void* beta, const float* state,
                                          void* o, float* inter_ssm, void* conv_window, void* act,
                                          void* workspace, size_t workspace_bytes,
                                          hipStream_t stream);

/* Accept step after a verify (PR#107 PR description: the per-token snapshots exist so the
 * caller can roll back to the accepted prefix). accepted [N] (device int32) holds a_n,
 * the number of tokens of sequence n that were kept, 1 <= a_n <= T. For each such n:
 *   state[cache_indices[n]]           <- inter_ssm[intermediate_state_indices[n], a_n - 1]
 *   conv_state[conv_state_indices[n]] <- conv_window[intermediate_state_indices[n], a_n - 1]
 * Bit copies. Sequences with a_n outside [1, T], and padding entries, are left alone.
 * p gives N, T, H, HV, K, V and in_dtype; pools as above (NULL = identity).
 * The rows a commit writes must be distinct among the sequences it commits (a_n in
 * [1, T], not padding): two of them with the same cache_indices row, or the same
 * conv_state_indices row, race, and that row then holds an unspecified mix of their
 * snapshots. Sequences that are not committed may share rows with anything. The index
 * arrays are device memory that the host does not read, so this is the caller's
 * contract and is not checked; NULL index arrays (the identity) are distinct by
 * construction. Host-side checks: NULL or misaligned pointers (KDA_ERR_NULL,
 * KDA_ERR_ALIGN), pool sizes (KDA_ERR_SHAPE), written ranges overlapping read ones or
 * each other (KDA_ERR_ALIAS); a rejected call launches nothing. */
kda_status kda_verify_commit(const kda_verify_params* p, const kda_pool_desc* pools,
                             const int32_t* accepted, const float* inter_ssm,
                             const void* conv_window, float* state, void* conv_state,
                             hipStream_t stream);

/* For callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc. kda_conv_verify_decode without a
 * workspace argument: the counters it needs (kda_workspace_bytes(p) bytes) live in a
 * static device array of the library, KDA_NOALLOC_SCRATCH_BYTES on each GPU the library
 * runs on, held until the process ends. Shapes that need more (N * H + 2 counter words
 * beyond it, e.g. N * H > 65534) return KDA_ERR_SCRATCH before any HIP call. Each call
 * first clears the counter words it uses with a small fill kernel on `stream` (no memset
 * node, so the call can be captured in a graph), then runs the same kernels as
 * kda_conv_verify_decode, with the same launch choice, results and validation; it calls
 * no allocating routine. The first call on a device looks up that device's copy of the
 * array (hipGetSymbolAddress, with the device current). Every call on a GPU shares its
 * array: calls that overlap on one GPU (two streams, two host threads) race on the
 * counters and may return wrong results, so a caller serialises them on one stream or
 * uses kda_conv_verify_decode with a workspace per stream. If the fill kernel launched
 * and the step's launch then fails, KDA_ERR_LAUNCH is returned after that fill. */
#define KDA_NOALLOC_SCRATCH_BYTES 262144
kda_status kda_conv_verify_decode_noalloc(const kda_verify_params* p, const void* mixed_qkv,
                                          const void* conv_weight, void* conv_state, const void* gate,
                                          const float* A_log, const float* dt_bias, const void* beta,
                                          const float* state, void* o, float* inter_ssm, void* conv_window,
                                          hipStream_t stream);

/* Static text for a kda_status value (never NULL). */
const char* kda_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* KDA_VERIFY_H */
