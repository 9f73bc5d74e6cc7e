// Fused causal-conv1d + Kimi Delta Attention (KDA) multi-token verify step for
// MI355X (gfx950, CDNA4), behind the C ABI of include/kda_verify.h.
//
// Operation: cuLA pull request page "[KDA] Fuse causal conv1d into MTP verify decode
// #107" (PR description): width-4 depthwise causal conv1d + SiLU over packed q/k/v,
// q/k L2 normalisation, softplus or safe decay gate, sigmoid beta, and the gated
// delta rule over T draft tokens with verify semantics (state read only, every
// token's state and conv window written, conv cache rolled in place).
//
// Design (our own, for gfx950; the page's CuTe kernels target NVIDIA parts):
//   * A unit of work is one (sequence n, value head hv, V-tile vt), done by one
//     workgroup (WG) that holds the fp32 K x VT state tile in VGPRs for all T tokens.
//     Three schedules: the grid (one WG per unit); the queue (as many WGs as are
//     resident at once, each pulling units from a counter in the workspace until none
//     are left, so that no XCD idles while another still has units); and the stream,
//     the queue with a fifth wave per WG, the producer, that draws the tickets and loads
//     the next unit's inputs and state tile straight into LDS while four compute waves
//     run the current one (the compute waves then issue no vector-memory read; the AUTO
//     choice for large batches). The WG's NW
//     wave64s split K: wave w owns rows [w*RW, (w+1)*RW). Inside a wave, LPR = VT/4
//     lanes span a row (one 16-byte vector of 4 columns each) and Q = 64/LPR
//     consecutive rows are covered by one instruction, so every state load and
//     snapshot store of a wave moves 64 x 16 contiguous bytes (two whole 512-byte rows
//     when VT = 128).
//   * Prologue (grid and queue): every input the WG needs besides the state (its q/k
//     channels, its v-column channels, their conv cache and weights, the gate row,
//     dt_bias, beta) is fetched with 16-byte loads into LDS; the 16-byte state loads are
//     issued right behind them and stay in flight through the conv / gate / l2norm math,
//     which all threads do from LDS. The stream's producer stages the same LDS layout.
//   * Token loop: the decay is folded into the two K-reductions,
//       u_j = sum_i (k_i a_i) S_ij,   w_j = sum_i (q_i a_i) S_ij,
//       d_j = beta (v_j - u_j),       o_j = w_j + (q.k) d_j,
//       S_ij <- a_i S_ij + k_i d_j,
//     one pass over the registers for both sums, cross-lane sums with DPP and the
//     gfx950 permlane16/32 swaps, one small LDS exchange of per-wave partial sums
//     (double-buffered, one barrier per token), then one pass to update and stream
//     the snapshot out with 16-byte non-temporal stores.
//   * K-sums follow one fixed tree in every tile shape (per wave: P partials of
//     RW/P rows each summed in row order, then a fixed pairing order over the
//     partials; then waves in index order), so the small and large variants are
//     bit-identical.
//   * The q/k part of conv_state is read by the g*NVT WGs of a (n, q/k head) group
//     and must be overwritten only after all of them read it (PR#107 description:
//     last-arrival counters). Each WG bumps a per-group counter once its reads have
//     landed; the one that sees the final count writes and re-zeroes the counter.
//     No WG ever waits on another.
// No MFMA: each token is rank-1 updates and matrix-vector products, bound by HBM.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <type_traits>

#include "kda_verify.h"
#define KDA_HOST_DEVICE __host__ __device__
#include "kda_queue.h"

// Counters of kda_conv_verify_decode_noalloc (the allocation-free entry point): one copy
// per GPU, held until the process ends. Host code never names this array in a kernel
// argument or a copy (on the host the name is only a stand-in): it uses the device address
// that hipGetSymbolAddress returns for the current device (kda::scratch_on_current_device).
static __device__ __align__(256) uint32_t scratch[KDA_NOALLOC_SCRATCH_BYTES / 4];

namespace kda {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ----------------------------------------------------------------------------------
// element types: raw storage of the input dtype (bf16 bits or fp32 bits)
// ----------------------------------------------------------------------------------
__device__ __forceinline__ float up(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }
__device__ __forceinline__ float up(uint32_t x) { return __uint_as_float(x); }

// Hardware transcendental forms (v_exp_f32, v_log_f32, v_rcp_f32, v_rsq_f32: about 1 ulp
// on the reduced argument). Overflow behaves: exp -> +inf, rcp(inf) -> 0, so the SiLU and
// sigmoid saturate to 0 / 1 without NaN.
__device__ __forceinline__ float exp_fast(float x) { return __builtin_amdgcn_exp2f(x * 1.44269504088896341f); }
__device__ __forceinline__ float log_fast(float x) { return __builtin_amdgcn_logf(x) * 0.69314718055994531f; }
__device__ __forceinline__ float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float rsqrt_fast(float x) { return __builtin_amdgcn_rsqf(x); }
__device__ __forceinline__ float sigmoid_fast(float x) { return rcp_fast(1.0f + exp_fast(-x)); }
__device__ __forceinline__ float silu_fast(float y) { return y * sigmoid_fast(y); }

// two floats -> packed bf16 pair (round to nearest even, NaN stays NaN): v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
}

template <typename R> struct OutVec;
template <> struct OutVec<uint16_t> {
  // 4 bf16 outputs -> one 8-byte store
  static __device__ __forceinline__ void store(void* base, size_t idx, float a, float b, float c, float d) {
    u32x2 v;
    v.x = bf16x2_rne(a, b);
    v.y = bf16x2_rne(c, d);
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(base) + idx) = v;
  }
};
template <> struct OutVec<uint32_t> {
  static __device__ __forceinline__ void store(void* base, size_t idx, float a, float b, float c, float d) {
    f32x4 v = {a, b, c, d};
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(base) + idx) = v;
  }
};

// ----------------------------------------------------------------------------------
// cross-lane all-reduce steps: x + x[lane ^ MASK], the same bits on both partners
// ----------------------------------------------------------------------------------
template <int MASK>
__device__ __forceinline__ float xor_sum(float x) {
  if constexpr (MASK == 32) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else if constexpr (MASK == 16) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else if constexpr (MASK == 8) {  // row_ror:8 inside a 16-lane row is lane ^ 8
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));
  } else if constexpr (MASK == 4) {  // ds_swizzle bit mode: and 0x1f, xor 4
    return x + __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x101f));
  } else if constexpr (MASK == 2) {  // quad_perm [2,3,0,1]
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4e, 0xf, 0xf, false));
  } else {
    static_assert(MASK == 1, "mask");  // quad_perm [1,0,3,2]
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xb1, 0xf, 0xf, false));
  }
}

// sum over the lanes that differ only in bits [log2(LO), 6) of the lane id
template <int LO>
__device__ __forceinline__ float lane_sum_from(float x) {
  if constexpr (LO <= 1) x = xor_sum<1>(x);
  if constexpr (LO <= 2) x = xor_sum<2>(x);
  if constexpr (LO <= 4) x = xor_sum<4>(x);
  if constexpr (LO <= 8) x = xor_sum<8>(x);
  if constexpr (LO <= 16) x = xor_sum<16>(x);
  if constexpr (LO <= 32) x = xor_sum<32>(x);
  return x;
}

// One 16-byte snapshot store with the chosen cache policy (vector memory only): the
// streaming (non-temporal) hint alone, or the streaming hint at device scope (nt sc1),
// which MI355X sweeps found faster on the large grids (see kStoreNTDev). The device-scope
// form is inline assembly, which the compiler's hazard tracking cannot see as a store: a
// 16-byte store's data registers must not be overwritten by VALU for two wait states after
// it on gfx950, so the statement supplies them itself (s_nop 1).
template <int STP>
__device__ __forceinline__ void store_snapshot(float* p, f32x4 v) {
  if constexpr (STP == 1)
    asm volatile("global_store_dwordx4 %0, %1, off nt sc1\n\ts_nop 1" ::"v"(p), "v"(v) : "memory");
  else
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
}

// Workgroups are handed to the 8 XCDs round-robin by blockIdx. Two orders of units over
// them, both bijections on [0, B):
//  * XCD ranges: each XCD works through one contiguous range of units, so the WGs sharing
//    an XCD's L2 stream through neighbouring state and snapshot addresses. Measured best
//    when a grid runs in several generations of workgroups (per-CU caps).
//  * pairs: pairs of neighbouring units are dealt to the XCDs in turn (units 2x and 2x + 1
//    of every 16 go to XCD x). Measured best when every workgroup of the grid is resident
//    at once: then all of them write the same token's snapshots at the same time, and
//    spreading each XCD's share over the whole batch sped those calls up by 1-9 % (the
//    512-unit four-token call by 11 %).
constexpr int kNXcd = 8;
__device__ __forceinline__ int xcd_order(int b, int B) {
  const int x = b % kNXcd, q = B / kNXcd, r = B % kNXcd;
  return x * q + (x < r ? x : r) + b / kNXcd;
}
__device__ __forceinline__ int pair_order(int b, int B) {
  constexpr int P = 2 * kNXcd;  // units per round of pairs
  if (b >= B - B % P) return b;  // the last partial round keeps its place
  const int x = b % kNXcd, i = b / kNXcd;
  return (i >> 1) * P + 2 * x + (i & 1);
}
enum UnitOrder { kOrderXcdRanges = 1, kOrderPairs = 2 };

// ----------------------------------------------------------------------------------
// kernel arguments
// ----------------------------------------------------------------------------------
struct Args {
  const void* mixed_qkv;
  const void* conv_weight;
  void* conv_state;
  const void* gate;
  const float* A_log;
  const float* dt_bias;
  const void* beta;
  const float* state;
  void* o;
  float* inter_ssm;
  void* conv_window;
  uint32_t* counters;
  // pool rows (NULL: the identity); a sequence with any index outside its pool is skipped
  const int32_t* cs_idx;
  const int32_t* st_idx;
  const int32_t* in_idx;
  int cs_slots, st_slots, in_slots;
  int N, T, H, HV, C;
  int g;      // HV / H
  int group;  // WGs reading one q/k head's conv cache: g * (V-tiles)
  int order;  // UnitOrder of the grid schedule
  int prefetch;  // stream schedule: StatePrefetch
  int gate_mode;
  float lower_bound, softplus_beta, softplus_threshold, scale, eps;
};

// Snapshot store cache policy: the streaming hint (nt), or the streaming hint with device
// scope (nt sc1). Timed on MI355X against plain device-scope stores (sc1) and system scope
// (nt sc0 sc1): nt sc1 moved large_batch from 80.3 % (nt) and 76.9 % (sc1) to 82.1 % of
// peak, and max_bandwidth from 80.8 % (sc1) to 82.7 %; system scope measured the same.
enum StorePolicy { kStoreNT = 0, kStoreNTDev = 1 };

// Partial-sum plan. A wave's P canonical partial sums of each column are paired in a
// fixed order of their index bits (1, 2, 0, then 3 when P = 16), the same for every tile
// shape, so that every variant forms the same sum. Index bits below LOGQ are lane bits
// (partner lane ^ (LPR << bit)), the others pair partials held by one lane. A lane level
// at lane distance 16 or 32 is a permlane swap that also halves the values each lane
// carries (one swap serves two sums); a shorter one is an all-reduce, after which the two
// lanes hold the same values (their distance bits form the DUP mask).
constexpr int plan_bit(int lv) { return lv == 0 ? 1 : lv == 1 ? 2 : lv == 2 ? 0 : 3; }
constexpr bool plan_halves(int lv, int logq, int lpr) {
  return plan_bit(lv) < logq && (lpr << plan_bit(lv)) >= 16;
}
constexpr int plan_nhalf(int logp, int logq, int lpr) {
  int c = 0;
  for (int l = 0; l < logp; ++l) c += plan_halves(l, logq, lpr) ? 1 : 0;
  return c;
}
constexpr int plan_dup(int logp, int logq, int lpr) {
  int m = 0;
  for (int l = 0; l < logp; ++l)
    if (plan_bit(l) < logq && !plan_halves(l, logq, lpr)) m |= lpr << plan_bit(l);
  return m;
}
constexpr int plan_half_mask(int j, int logp, int logq, int lpr) {  // lane bit of halving j
  for (int l = 0; l < logp; ++l)
    if (plan_halves(l, logq, lpr) && j-- == 0) return lpr << plan_bit(l);
  return 0;
}

// PRE_ = 1: the unfused form of the step. The conv + SiLU ran in a separate kernel and
// mixed_qkv holds its fp32 activations; this kernel only stages them (no conv cache, no
// taps, no conv-window or conv-state writes).
// G_ column groups: a WG covers WT = G * VT columns of V with G groups of NW waves, group g
// taking columns [g * VT, (g + 1) * VT) exactly as a one-group WG of VT columns would (same
// K split, same sum tree, same bits); the staging, conv, gate and l2norm are shared.
template <typename R, int K_, int V_, int VT_, int NW_, int TMAX_, int STP_ = kStoreNT, int PRE_ = 0, int G_ = 1>
struct Cfg {
  static constexpr int K = K_, V = V_, VT = VT_, NW = NW_, TMAX = TMAX_, STP = STP_, PRE = PRE_, G = G_;
  static constexpr int WT = G * VT;      // V columns per WG
  static constexpr int NWT = G * NW;     // waves per WG
  static constexpr int NTHR = NWT * 64;
  static constexpr int NVT = V / WT;     // WGs per (n, hv)
  static constexpr int RW = K / NW;      // K rows per wave
  static constexpr int LPR = VT / 4;     // lanes across one row of the tile
  static constexpr int Q = 64 / LPR;     // rows one wave instruction covers
  static constexpr int RPL = RW / Q;     // rows per lane
  static constexpr int P = K >= 64 ? 8 : 16;  // canonical partial sums per wave and column
  static constexpr int M = P / Q;        // partials a lane holds
  static constexpr int LOGQ = Q == 1 ? 0 : Q == 2 ? 1 : Q == 4 ? 2 : Q == 8 ? 3 : 4;
  static constexpr int LOGP = P == 8 ? 3 : 4;
  static constexpr int NCH = 2 * K + WT;        // channels a WG stages: q, k, its v columns
  static constexpr int E16 = 16 / (int)sizeof(R);  // elements per 16-byte vector
  using XR = typename std::conditional<PRE_ != 0, uint32_t, R>::type;  // staged token rows
  static constexpr int XE16 = 16 / (int)sizeof(XR);
  static_assert(V % WT == 0 && VT % 4 == 0 && 64 % LPR == 0 && K % NW == 0 && NTHR <= 1024, "tile shape");
  static_assert(RW % Q == 0 && P % Q == 0 && RPL % M == 0 && (1 << LOGQ) == Q && RW % P == 0, "rows");
  static_assert(K % E16 == 0 && VT % E16 == 0 && K % 4 == 0 && K <= 128, "vector widths");
  // the partial-sum plan of this shape
  static constexpr int sum_bit(int lv) { return plan_bit(lv); }
  static constexpr bool halves(int lv) { return plan_halves(lv, LOGQ, LPR); }
  static constexpr int NHALF = plan_nhalf(LOGP, LOGQ, LPR);
  static constexpr int DUP = plan_dup(LOGP, LOGQ, LPR);
  static constexpr int half_mask(int j) { return plan_half_mask(j, LOGP, LOGQ, LPR); }
  static constexpr int NOUT = 8 >> NHALF;  // (u|w, column) sums a lane ends with
  static_assert(NHALF <= 3, "halving levels");
  // 16-byte vectors staged per WG at T = TMAX
  static constexpr int MAX_CHUNKS = TMAX * NCH / XE16 + 3 * NCH / E16 + 4 * NCH / E16 + TMAX * K / E16 + K / 4;
  static constexpr int MAXC = (MAX_CHUNKS + NTHR - 1) / NTHR;
};

// Halving step across lanes l and l ^ MASK (MASK 16 or 32): the lane with that bit clear
// returns a[l] + a[l ^ MASK], the other b[l] + b[l ^ MASK]. One swap serves two sums.
template <int MASK>
__device__ __forceinline__ float swap_sum(float a, float b) {
  static_assert(MASK == 16 || MASK == 32, "swap mask");
  const auto r = MASK == 32 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false)
                            : __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Reduce a lane's partials acc[m][label] (label = 4 * (w ? 1 : 0) + column) over the P
// canonical partials of a wave, level LV of the pairing order onward. CNT labels are live;
// DONE holds the partial-index bits already summed within the lane.
template <class CF, int LV, int CNT, int DONE>
__device__ __forceinline__ void reduce_partials(float (&acc)[CF::M][8]) {
  if constexpr (LV < CF::LOGP) {
    constexpr int bit = CF::sum_bit(LV);
    if constexpr (bit >= CF::LOGQ) {  // both partners in this lane
      constexpr int mb = 1 << (bit - CF::LOGQ);
#pragma unroll
      for (int m = 0; m < CF::M; ++m)
        if ((m & DONE) == 0 && (m & mb) == 0)
#pragma unroll
          for (int l = 0; l < CNT; ++l) acc[m][l] += acc[m | mb][l];
      reduce_partials<CF, LV + 1, CNT, DONE | mb>(acc);
    } else if constexpr (CF::halves(LV)) {  // partner lane ^ mask, split the labels
      constexpr int mask = CF::LPR << bit, h = CNT / 2;
#pragma unroll
      for (int m = 0; m < CF::M; ++m)
        if ((m & DONE) == 0)
#pragma unroll
          for (int l = 0; l < h; ++l) acc[m][l] = swap_sum<mask>(acc[m][l], acc[m][l + h]);
      reduce_partials<CF, LV + 1, h, DONE>(acc);
    } else {  // partner lane ^ mask, both keep every label
      constexpr int mask = CF::LPR << bit;
#pragma unroll
      for (int m = 0; m < CF::M; ++m)
        if ((m & DONE) == 0)
#pragma unroll
          for (int l = 0; l < CNT; ++l) acc[m][l] = xor_sum<mask>(acc[m][l]);
      reduce_partials<CF, LV + 1, CNT, DONE>(acc);
    }
  }
}

template <class CF, typename R>
struct alignas(16) Smem {
  f32x4 row[CF::TMAX * CF::K];        // per token, per K row: {k*a, q*a, a, k} (q scaled)
  float vs[CF::TMAX * CF::WT];        // SiLU(conv(v)) of the WG's columns
  f32x4 part[2][CF::NWT][2][CF::LPR];  // per-wave partial sums (u, w), double-buffered by token
  float betas[CF::TMAX];
  float qk[CF::TMAX];
  alignas(16) typename CF::XR xs[CF::TMAX * CF::NCH];  // raw new tokens, [t][local channel]
  alignas(16) R cs[3 * CF::NCH];         // raw conv cache, [local channel][3]
  alignas(16) R ws[4 * CF::NCH];         // conv taps, [local channel][4]
  alignas(16) R gs[CF::TMAX * CF::K];    // raw gate, [t][K]
  // raw conv window of every token, laid out as its output row: [t][local channel][3]
  alignas(16) R win[CF::PRE ? 8 : CF::TMAX * CF::NCH * 3];
  alignas(16) float dtb[CF::K];
  uint32_t bs[CF::TMAX];  // raw beta of each token, widened to 32 bits (bf16 in the low half)
  int last;
  uint32_t next[2];  // queue schedule: the ticket for the next unit, by iteration parity
};

template <class CF>
__device__ __forceinline__ int row_slot(int t, int i) {
  return t * CF::K + i;
}

// global channel of local staged channel lc (q block, k block, then this WG's v columns)
template <class CF>
__device__ __forceinline__ int gchan(int lc, int h, int H, int hv, int vt) {
  if (lc < CF::K) return h * CF::K + lc;
  if (lc < 2 * CF::K) return H * CF::K + h * CF::K + (lc - CF::K);
  return 2 * H * CF::K + hv * CF::V + vt * CF::WT + (lc - 2 * CF::K);
}

// Where a unit sits: its sequence, value head, q/k head, V-tile, and its pool rows (conv
// cache; snapshots and windows).
struct UnitAt {
  int n, hv, h, vt, cs_row, in_row;
};

// Phases 1a and 1b of a unit, from the inputs staged in LDS: conv + SiLU of every staged
// channel (and the raw windows left for the copies), then the decay and beta of each token.
template <class CF, typename R>
__device__ __forceinline__ void conv_and_gates(const Args& a, Smem<CF, R>& s, const bool qk_owner, const float alog) {
  constexpr int K = CF::K, NCH = CF::NCH, NTHR = CF::NTHR;
  const int tid = threadIdx.x;
  const int T = a.T;
  __builtin_assume(T >= 1 && T <= CF::TMAX);
  // ---------------- phase 1a: conv + SiLU, one task per pair of staged channels, sliding
  // over the tokens (taps and the three cached inputs read once per channel); the raw
  // window each token leaves behind, e[t+1..t+3], is staged in LDS in the layout of its
  // output row, two channels (six values) per write
  // q/k windows are written out by one WG of the group (all tokens) and the rolled q/k
  // cache by the last WG to count in (the last token's window): a WG stages only those
  for (int pr = tid; pr < NCH / 2; pr += NTHR) {
    const int ch = 2 * pr;  // the pair never straddles the q | k | v blocks (all even)
    const int t_stage = ch < 2 * K && !qk_owner ? T - 1 : 0;  // first token whose window is staged
    // destination of (channel ch, token t); channel ch + 1 sits `cstride` floats further
    float* dp;
    int dstride, cstride;
    if (ch < K) {
      dp = reinterpret_cast<float*>(&s.row[ch]) + 1;
      dstride = 4 * K;
      cstride = 4;
    } else if (ch < 2 * K) {
      dp = reinterpret_cast<float*>(&s.row[ch - K]);
      dstride = 4 * K;
      cstride = 4;
    } else {
      dp = &s.vs[ch - 2 * K];
      dstride = CF::WT;
      cstride = 1;
    }
    if constexpr (CF::PRE) {  // already convolved and activated
#pragma unroll
      for (int t = 0; t < CF::TMAX; ++t)
        if (t < T) {
          dp[t * dstride] = up(s.xs[t * NCH + ch]);
          dp[t * dstride + cstride] = up(s.xs[t * NCH + ch + 1]);
        }
    } else {
      float w[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) w[j] = up(s.ws[ch * 4 + j]);
      // raw inputs e[t..t+3] of both channels: the three cached ones, then the new tokens
      R a0 = s.cs[ch * 3 + 0], a1 = s.cs[ch * 3 + 1], a2 = s.cs[ch * 3 + 2];
      R b0 = s.cs[ch * 3 + 3], b1 = s.cs[ch * 3 + 4], b2 = s.cs[ch * 3 + 5];
#pragma unroll
      for (int t = 0; t < CF::TMAX; ++t) {
        if (t < T) {
          const R a3 = s.xs[t * NCH + ch], b3 = s.xs[t * NCH + ch + 1];
          const float ya = fmaf(w[3], up(a3), fmaf(w[2], up(a2), fmaf(w[1], up(a1), w[0] * up(a0))));
          const float yb = fmaf(w[7], up(b3), fmaf(w[6], up(b2), fmaf(w[5], up(b1), w[4] * up(b0))));
          dp[t * dstride] = silu_fast(ya);
          dp[t * dstride + cstride] = silu_fast(yb);
          if (t >= t_stage) {
            R* wr = &s.win[(t * NCH + ch) * 3];
            wr[0] = a1;
            wr[1] = a2;
            wr[2] = a3;
            wr[3] = b1;
            wr[4] = b2;
            wr[5] = b3;
          }
          a0 = a1;
          a1 = a2;
          a2 = a3;
          b0 = b1;
          b1 = b2;
          b2 = b3;
        }
      }
    }
  }

  // ---------------- phase 1b: gate -> alpha, beta
  {
    const float eA = exp_fast(alog);
    const float inv_sb = rcp_fast(a.softplus_beta);
    for (int gi = tid; gi < T * K; gi += NTHR) {
      const int t = gi / K, i = gi - (gi / K) * K;
      const float gam = up(s.gs[gi]) + s.dtb[i];
      float ld;
      if (a.gate_mode == KDA_GATE_SOFTPLUS) {
        const float bx = a.softplus_beta * gam;
        float sp;
        if (bx <= a.softplus_threshold)
          sp = log_fast(1.0f + exp_fast(bx)) * inv_sb;
        else
          sp = gam;  // linear tail; the exponential is not formed here
        ld = -eA * sp;
      } else {
        ld = a.lower_bound * sigmoid_fast(eA * gam);
      }
      s.row[row_slot<CF>(t, i)].z = exp_fast(ld);
    }
    if (tid < T) s.betas[tid] = sigmoid_fast(up((R)s.bs[tid]));
  }

}

// Phase 2a of a unit: q/k l2norm per token (one wave per token), decay folded in.
template <class CF, typename R>
__device__ __forceinline__ void l2norm_tokens(const Args& a, Smem<CF, R>& s) {
  constexpr int K = CF::K;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int T = a.T;
  __builtin_assume(T >= 1 && T <= CF::TMAX);
  // ---------------- phase 2a: q/k l2norm per token (one wave per token), fold alpha in
  for (int t = wave; t < T; t += CF::NWT) {
    float kx[2], qx[2];
    float sk = 0.f, sq = 0.f, sqk = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = lane + 64 * u;
      kx[u] = qx[u] = 0.f;
      if (i < K) {
        const f32x4 r = s.row[row_slot<CF>(t, i)];
        kx[u] = r.x;
        qx[u] = r.y;
      }
      sk = fmaf(kx[u], kx[u], sk);
      sq = fmaf(qx[u], qx[u], sq);
      sqk = fmaf(qx[u], kx[u], sqk);
    }
    sk = lane_sum_from<1>(sk);
    sq = lane_sum_from<1>(sq);
    sqk = lane_sum_from<1>(sqk);
    const float rk = rsqrt_fast(sk + a.eps);
    const float rq = a.scale * rsqrt_fast(sq + a.eps);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = lane + 64 * u;
      if (i < K) {
        f32x4& r = s.row[row_slot<CF>(t, i)];
        const float al = r.z;
        const float kh = kx[u] * rk, qh = qx[u] * rq;
        r = f32x4{kh * al, qh * al, al, kh};
      }
    }
    if (lane == 0) s.qk[t] = sqk * rk * rq;
  }

}

template <class CF, typename R>
__device__ __forceinline__ void grid_raw_copies(const Args& a, Smem<CF, R>& s, const UnitAt& u, const bool qk_owner) {
  constexpr int K = CF::K, NCH = CF::NCH, E16 = CF::E16, NTHR = CF::NTHR;
  const int tid = threadIdx.x;
  const int T = a.T, H = a.H, C = a.C;
  const int h = u.h, hv = u.hv, vt = u.vt, cs_row = u.cs_row, in_row = u.in_row;
  R* cstate = static_cast<R*>(a.conv_state);
  // ---------------- grid schedule: every raw copy of the unit before the first token's
  // sums (the conv window of each token, then the rolled conv cache, with the same owners
  // as the queue's per-token copies in the token loop). A grid WG runs one unit and exits;
  // with these stores here it ends with its last snapshot instead of a tail of copies, which
  // measured 0.6-2.8 % faster on grids of 512-1536 units, same bits. Every thread issues the
  // same number of 16-byte stores (a slot past the end repeats the last vector: the same
  // bytes to the same address), so the count in flight stays known to the compiler and the
  // token loop waits on none of them. Issued here on the queue schedule they cost 1-3 %
  // (measured): there the copies of a unit overlap the next unit's loads anyway, and here
  // they delay its first snapshot.
  if constexpr (!CF::PRE) {
    constexpr int VQK = 3 * K / E16;
    constexpr int VV = 3 * CF::WT / E16;
    constexpr int MAXR = CF::TMAX * (2 * VQK + VV) + VV + 2 * VQK;
    constexpr int NR = (MAXR + NTHR - 1) / NTHR;
    const int nqk = qk_owner ? 2 * VQK : 0;
    const int per_t = nqk + VV;
    const int nwin = T * per_t;
    const int tot = nwin + VV + (s.last ? 2 * VQK : 0);
    R* cw = static_cast<R*>(a.conv_window);
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      int q = tid + k * NTHR;
      q = q < tot ? q : tot - 1;
      int t, lc0, m;
      size_t off;
      R* base;
      if (q < nwin) {
        t = q / per_t;
        const int r = q - t * per_t;
        if (r < nqk) {
          const int blk = r / VQK;
          m = r - blk * VQK;
          lc0 = blk * K;
        } else {
          m = r - nqk;
          lc0 = 2 * K;
        }
        base = cw;
        off = (((size_t)in_row * T + t) * C + gchan<CF>(lc0, h, H, hv, vt)) * 3;
      } else {
        int r = q - nwin;
        t = T - 1;
        if (r < VV) {
          m = r;
          lc0 = 2 * K;
        } else {
          r -= VV;
          const int blk = r / VQK;
          m = r - blk * VQK;
          lc0 = blk * K;
        }
        base = cstate;
        off = ((size_t)cs_row * C + gchan<CF>(lc0, h, H, hv, vt)) * 3;
      }
      *reinterpret_cast<u32x4*>(base + off + m * E16) =
          *reinterpret_cast<const u32x4*>(&s.win[(t * NCH + lc0) * 3 + m * E16]);
    }
  }

}

// The token loop of a unit: the gated delta-rule update of the state tile S held in
// registers, o, the snapshot of every token, and (queue schedules) each token's raw copies.
template <class CF, typename R, bool QUEUE>
__device__ __forceinline__ void token_loop(const Args& a, Smem<CF, R>& s, f32x4 (&S)[CF::RPL], const UnitAt& u,
                                           const bool qk_owner) {
  constexpr int K = CF::K, V = CF::V, NCH = CF::NCH, E16 = CF::E16, NTHR = CF::NTHR;
  constexpr int RPL = CF::RPL, VT = CF::VT, Q = CF::Q, LPR = CF::LPR, M = CF::M;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int T = a.T, H = a.H, HV = a.HV, C = a.C;
  __builtin_assume(T >= 1 && T <= CF::TMAX);
  const int n = u.n, hv = u.hv, h = u.h, vt = u.vt, cs_row = u.cs_row, in_row = u.in_row;
  R* cstate = static_cast<R*>(a.conv_state);
  const int grp = wave / CF::NW, wv = wave - grp * CF::NW;
  const int c4 = lane % LPR, qq = lane / LPR;
  const int col = vt * CF::WT + grp * VT + c4 * 4;
  const int row0 = wv * CF::RW + qq;
  const size_t KV = (size_t)K * V;
  // ---------------- token loop
  float* snap = a.inter_ssm + (size_t)row0 * V + col;
  for (int t = 0; t < T; ++t) {
    const f32x4* rw = &s.row[t * K + row0];
    // per-lane partials: rows row0 + Q*r, partial m = r % M, rows of a partial in order;
    // label c is column c of u, label 4 + c column c of w
    float acc[M][8];
    // a_i and k_i of the lane's rows, kept in registers for the update when there are few
    constexpr bool KEEP = RPL <= 8;
    float ra[KEEP ? RPL : 1], rk[KEEP ? RPL : 1];
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      const int m = r % M;
      const f32x4 rr = rw[r * Q];
      const f32x4 sv = S[r];
      if constexpr (KEEP) {
        ra[r] = rr.z;
        rk[r] = rr.w;
      }
      if (r < M) {
        acc[m][0] = rr.x * sv.x; acc[m][1] = rr.x * sv.y; acc[m][2] = rr.x * sv.z; acc[m][3] = rr.x * sv.w;
        acc[m][4] = rr.y * sv.x; acc[m][5] = rr.y * sv.y; acc[m][6] = rr.y * sv.z; acc[m][7] = rr.y * sv.w;
      } else {
        acc[m][0] = fmaf(rr.x, sv.x, acc[m][0]); acc[m][1] = fmaf(rr.x, sv.y, acc[m][1]);
        acc[m][2] = fmaf(rr.x, sv.z, acc[m][2]); acc[m][3] = fmaf(rr.x, sv.w, acc[m][3]);
        acc[m][4] = fmaf(rr.y, sv.x, acc[m][4]); acc[m][5] = fmaf(rr.y, sv.y, acc[m][5]);
        acc[m][6] = fmaf(rr.y, sv.z, acc[m][6]); acc[m][7] = fmaf(rr.y, sv.w, acc[m][7]);
      }
    }
    reduce_partials<CF, 0, 8, 0>(acc);
    // wave partials through LDS, then waves summed in index order; the lanes left holding a
    // distinct group of NOUT labels write it
    const int buf = t & 1;
    if ((lane & CF::DUP) == 0) {
      int lab = 0;
      if constexpr (CF::NHALF >= 1) lab += (lane & CF::half_mask(0)) ? 4 : 0;
      if constexpr (CF::NHALF >= 2) lab += (lane & CF::half_mask(1)) ? 2 : 0;
      if constexpr (CF::NHALF >= 3) lab += (lane & CF::half_mask(2)) ? 1 : 0;
      float* pp = reinterpret_cast<float*>(&s.part[buf][wave][lab >> 2][c4]) + (lab & 3);
      if constexpr (CF::NOUT == 8) {
        s.part[buf][wave][0][c4] = f32x4{acc[0][0], acc[0][1], acc[0][2], acc[0][3]};
        s.part[buf][wave][1][c4] = f32x4{acc[0][4], acc[0][5], acc[0][6], acc[0][7]};
      } else if constexpr (CF::NOUT == 4) {
        *reinterpret_cast<f32x4*>(pp) = f32x4{acc[0][0], acc[0][1], acc[0][2], acc[0][3]};
      } else if constexpr (CF::NOUT == 2) {
        *reinterpret_cast<float2*>(pp) = make_float2(acc[0][0], acc[0][1]);
      } else {
        *pp = acc[0][0];
      }
    }
    __syncthreads();
    const int w0 = grp * CF::NW;  // the group's first wave
    f32x4 uu = s.part[buf][w0][0][c4], ww = s.part[buf][w0][1][c4];
    if constexpr (CF::NW == 2) {
      uu += s.part[buf][w0 + 1][0][c4];
      ww += s.part[buf][w0 + 1][1][c4];
    } else if constexpr (CF::NW == 4) {
      uu = (uu + s.part[buf][w0 + 1][0][c4]) + (s.part[buf][w0 + 2][0][c4] + s.part[buf][w0 + 3][0][c4]);
      ww = (ww + s.part[buf][w0 + 1][1][c4]) + (s.part[buf][w0 + 2][1][c4] + s.part[buf][w0 + 3][1][c4]);
    } else {
      static_assert(CF::NW == 1, "waves per WG");
    }
    const f32x4 vv = *reinterpret_cast<const f32x4*>(&s.vs[t * CF::WT + grp * VT + c4 * 4]);
    const float bt = s.betas[t], qk = s.qk[t];
    float d[4];
    d[0] = bt * (vv.x - uu.x);
    d[1] = bt * (vv.y - uu.y);
    d[2] = bt * (vv.z - uu.z);
    d[3] = bt * (vv.w - uu.w);
    const size_t nth = (size_t)(n * T + t) * HV + hv;
    const size_t ith = ((size_t)in_row * T + t) * HV + hv;
    if (wv == 0 && qq == 0)
      OutVec<R>::store(a.o, nth * V + col, fmaf(qk, d[0], ww.x), fmaf(qk, d[1], ww.y),
                       fmaf(qk, d[2], ww.z), fmaf(qk, d[3], ww.w));
    // S_ij <- a_i S_ij + k_i d_j, then stream the snapshot out
    float* dst = snap + ith * KV;
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      float al, kr;
      if constexpr (KEEP) {
        al = ra[r];
        kr = rk[r];
      } else {
        const f32x4 rr = rw[r * Q];
        al = rr.z;
        kr = rr.w;
      }
      // a_i S_ij rounded, then + k_i d_j fused: the product lands in S's own register
      f32x4 sv = S[r];
      sv.x = fmaf(kr, d[0], al * sv.x);
      sv.y = fmaf(kr, d[1], al * sv.y);
      sv.z = fmaf(kr, d[2], al * sv.z);
      sv.w = fmaf(kr, d[3], al * sv.w);
      S[r] = sv;
      store_snapshot<CF::STP>(dst + (size_t)r * Q * V, sv);
    }

    // queue schedule: the raw copies of this token, after its snapshot (no load follows, so
    // nothing ever waits on them): 16-byte vectors of the window rows staged in LDS. The
    // conv window of the v columns always and of q/k by one WG per group; after the last
    // token the rolled conv cache (that token's window) of the v columns (read only by this
    // WG), and of the shared q/k channels by the last WG of the group to count in (every
    // other WG of the group counted itself only after its reads had landed)
    if constexpr (!CF::PRE && QUEUE) {
      constexpr int VQK = 3 * K / E16;  // vectors per token of the q or the k block
      constexpr int VV = 3 * CF::WT / E16;  // vectors per token of this WG's v block
      const int nqk = qk_owner ? 2 * VQK : 0;
      const int nwin = nqk + VV;
      const int tot = nwin + (t == T - 1 ? VV + (s.last ? 2 * VQK : 0) : 0);
      R* cw = static_cast<R*>(a.conv_window);
      for (int q = tid; q < tot; q += NTHR) {
        const bool to_cache = q >= nwin;
        int r = to_cache ? q - nwin : q;
        int lc0, m;  // first local channel of the block, vector within the block
        if (to_cache ? r < VV : r >= nqk) {
          m = to_cache ? r : r - nqk;
          lc0 = 2 * K;
        } else {
          if (to_cache) r -= VV;
          const int blk = r / VQK;
          m = r - blk * VQK;
          lc0 = blk * K;
        }
        const int gc0 = gchan<CF>(lc0, h, H, hv, vt);
        R* wdst = to_cache ? cstate + ((size_t)cs_row * C + gc0) * 3 : cw + (((size_t)in_row * T + t) * C + gc0) * 3;
        *reinterpret_cast<u32x4*>(wdst + m * E16) =
            *reinterpret_cast<const u32x4*>(&s.win[(t * NCH + lc0) * 3 + m * E16]);
      }
    }
  }
}

// One (sequence, value head, V-tile) unit of the step, by the whole workgroup. Under the
// queue schedule (QUEUE) thread 0 also takes a ticket for the workgroup's next unit as
// the unit starts and leaves it in s.next[slot] before the first barrier.
template <class CF, typename R, bool QUEUE>
__device__ __forceinline__ void verify_unit(const Args& a, Smem<CF, R>& s, const int lb, const int slot) {
  constexpr int K = CF::K, V = CF::V, NCH = CF::NCH, E16 = CF::E16, NTHR = CF::NTHR;
  constexpr int RPL = CF::RPL, VT = CF::VT, Q = CF::Q, LPR = CF::LPR;

  const int tid = threadIdx.x;
  // The ticket is drawn by thread 0 and read only by thread 0, on the same path, so no
  // other lane ever reads it. It gets no initial value on purpose: one would make the
  // compiler set the register at the top of every unit, and that write waits first for
  // every store of the previous unit still in flight (measured; a zero, an empty asm
  // defining it and __builtin_nondeterministic_value all do).
  uint32_t ticket;
  if constexpr (QUEUE)
    if (tid == 0)
      ticket = __hip_atomic_fetch_add(a.counters + (size_t)a.N * a.H, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int wave = tid >> 6, lane = tid & 63;
  const int T = a.T, H = a.H, HV = a.HV, C = a.C;
  __builtin_assume(T >= 1 && T <= CF::TMAX);
  const int vt = lb % CF::NVT;
  const int unit = lb / CF::NVT;  // n * HV + hv
  const int hv = unit % HV, n = unit / HV;
  const int h = hv / a.g;
  // pool rows of this sequence: conv cache, state, and the snapshot / window pools
  const int cs_row = a.cs_idx ? a.cs_idx[n] : n;
  const int st_row = a.st_idx ? a.st_idx[n] : n;
  const int in_row = a.in_idx ? a.in_idx[n] : n;
  if (cs_row < 0 || cs_row >= a.cs_slots || st_row < 0 || st_row >= a.st_slots || in_row < 0 ||
      in_row >= a.in_slots) {
    // padding entry: the whole unit (and its group) skips, nothing is read or written
    if constexpr (QUEUE)
      if (tid == 0) s.next[slot] = ticket;
    return;
  }

  const typename CF::XR* __restrict__ xq = static_cast<const typename CF::XR*>(a.mixed_qkv);
  const R* __restrict__ wq = static_cast<const R*>(a.conv_weight);
  R* cstate = static_cast<R*>(a.conv_state);
  const R* __restrict__ gq = static_cast<const R*>(a.gate);
  const R* __restrict__ bq = static_cast<const R*>(a.beta);

  // ---------------- prologue: issue every 16-byte load of the WG's small inputs
  const int PA = NCH / CF::XE16;
  const int nA = T * PA;              // new tokens
  const int nB = CF::PRE ? 0 : 3 * NCH / E16;  // conv cache
  const int nC = CF::PRE ? 0 : 4 * NCH / E16;  // conv taps
  const int nD = T * K / E16;         // gate
  const int nE = K / 4;               // dt_bias (fp32)
  const int total = nA + nB + nC + nD + nE;
  u32x4 vals[CF::MAXC];
  int dsts[CF::MAXC];
  char* lds = reinterpret_cast<char*>(&s);
  const float alog = a.A_log[hv];
  // Every slot loads unconditionally (a slot past the end re-reads the last vector and
  // is not stored), so the loads issue back to back with no wait between them.
#pragma unroll
  for (int k = 0; k < CF::MAXC; ++k) {
    const int cv = tid + k * NTHR;
    int ci = cv < total ? cv : total - 1;
    const void* src;
    int dst;
    if (ci < nA) {
      const int t = ci / PA, pe = (ci - t * PA) * CF::XE16;
      src = xq + (size_t)(n * T + t) * C + gchan<CF>(pe, h, H, hv, vt);
      dst = (int)((char*)&s.xs[t * NCH + pe] - lds);
    } else if ((ci -= nA) < nB) {
      const int e = ci * E16, lc = e / 3;
      src = cstate + ((size_t)cs_row * C + gchan<CF>(lc, h, H, hv, vt)) * 3 + (e - lc * 3);
      dst = (int)((char*)&s.cs[e] - lds);
    } else if ((ci -= nB) < nC) {
      const int e = ci * E16, lc = e / 4;
      src = wq + (size_t)gchan<CF>(lc, h, H, hv, vt) * 4 + (e - lc * 4);
      dst = (int)((char*)&s.ws[e] - lds);
    } else if ((ci -= nC) < nD) {
      const int e = ci * E16, t = e / K;
      src = gq + ((size_t)(n * T + t) * HV + hv) * K + (e - t * K);
      dst = (int)((char*)&s.gs[e] - lds);
    } else {
      ci -= nD;
      src = a.dt_bias + (size_t)hv * K + ci * 4;
      dst = (int)((char*)&s.dtb[ci * 4] - lds);
    }
    vals[k] = *reinterpret_cast<const u32x4*>(src);
    dsts[k] = cv < total ? dst : -1;
  }
  const R bval = bq[(size_t)(n * T + (tid < T ? tid : T - 1)) * HV + hv];

  // ---------------- state tile: 16-byte loads, left in flight through the prologue math
  const int grp = wave / CF::NW, wv = wave - grp * CF::NW;  // column group, wave in the group
  const int c4 = lane % LPR, qq = lane / LPR;
  const int col = vt * CF::WT + grp * VT + c4 * 4;
  const int row0 = wv * CF::RW + qq;  // this lane's rows: row0 + Q * r
  const size_t KV = (size_t)K * V;
  const float* sp = a.state + ((size_t)st_row * HV + hv) * KV + (size_t)row0 * V + col;
  f32x4 S[RPL];
#pragma unroll
  for (int r = 0; r < RPL; ++r)
    S[r] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(sp + (size_t)r * Q * V));

#pragma unroll
  for (int k = 0; k < CF::MAXC; ++k)
    if (dsts[k] >= 0) *reinterpret_cast<u32x4*>(lds + dsts[k]) = vals[k];
  if (tid < T) s.bs[tid] = (uint32_t)bval;
  if constexpr (QUEUE) {
    // the ticket was issued before the staged loads just waited for, so it has landed
    if (tid == 0) s.next[slot] = ticket;
  }
  __syncthreads();  // B0: staged inputs visible; this WG's conv-cache reads have landed

  // q/k conv-cache ownership: count this WG in now (its reads have landed); the count
  // is read only after the prologue math, so nothing waits on the atomic until then.
  uint32_t prev = 0;
  if (!CF::PRE && tid == 0 && a.group > 1)
    prev = __hip_atomic_fetch_add(a.counters + (size_t)n * H + h, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  const bool qk_owner = (hv % a.g == 0) && vt == 0;
  conv_and_gates<CF, R>(a, s, qk_owner, alog);
  __syncthreads();  // B1
  l2norm_tokens<CF, R>(a, s);
  if (tid == 0) {
    const bool last = a.group <= 1 || prev == (uint32_t)(a.group - 1);
    if (last && a.group > 1)
      __hip_atomic_store(a.counters + (size_t)n * H + h, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s.last = last;
  }
  __syncthreads();  // B2

  const UnitAt u{n, hv, h, vt, cs_row, in_row};
  if constexpr (!QUEUE) grid_raw_copies<CF, R>(a, s, u, qk_owner);
  token_loop<CF, R, QUEUE>(a, s, S, u, qk_owner);
}

// Grid schedule: one workgroup per unit; the hardware starts each workgroup as a slot on
// a CU frees up, and hands workgroups to the XCDs round-robin, so every XCD gets the same
// number of units whatever its speed.
template <class CF, typename R>
__global__ __launch_bounds__(CF::NTHR) void kda_verify_kernel(const Args a) {
  __shared__ Smem<CF, R> s;
  const int b = blockIdx.x, B = gridDim.x;
  verify_unit<CF, R, false>(a, s, a.order == kOrderPairs ? pair_order(b, B) : xcd_order(b, B), 0);
}

// Queue schedule: only as many workgroups as are resident at once. Each takes one unit
// of the first round by blockIdx, then keeps pulling the next unit from a counter in the
// workspace (units handed out past the first round) until the units run out, so an XCD
// that runs faster takes more of them, and no workgroup launch sits between units. The
// last workgroup to leave zeroes the counter and the leave count for the next call: every
// workgroup drew its last ticket, and saw it past the end, before it counted itself out.
template <class CF, typename R>
__global__ __launch_bounds__(CF::NTHR) void kda_verify_queue_kernel(const Args a) {
  __shared__ Smem<CF, R> s;
  const int units = a.N * a.HV * CF::NVT;
  const int G = gridDim.x;  // <= units
  int lb = xcd_order(blockIdx.x, G);
  for (int it = 0; lb >= 0; ++it) {
    verify_unit<CF, R, true>(a, s, lb, it & 1);
    __syncthreads();  // the unit's LDS reads are done before the next unit stages inputs
    lb = kda_queue_unit(s.next[it & 1], units, G);
  }
  if (threadIdx.x == 0) {
    uint32_t* q = a.counters + (size_t)a.N * a.H;
    const uint32_t left = __hip_atomic_fetch_add(q + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (left == (uint32_t)G - 1) {
      __hip_atomic_store(q, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(q + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Stream schedule: the queue schedule with the loads taken off the compute waves. A fifth
// wave, the producer, pulls the units from the counter and loads each one's inputs and
// state tile straight into LDS (LDS-direct loads) while the four compute waves run the
// unit before it. The compute waves then issue no vector-memory read at all; on CDNA the
// vector-memory counter of a wave completes in issue order, so a load of theirs would wait
// for every snapshot store they issued before it, and this is what made a queue unit's
// staged phase longer than a grid unit's. The producer's counter holds only its own loads
// and atomics, and it waits on them only before the barrier that hands the next unit over,
// with the whole token loop of the current unit as slack.
//
// When the producer issues the next unit's state tile:
//   kPrefetchAfterConv:  with its other inputs, once the compute waves finished the conv and
//                        gates of the current unit (LDS staging free);
//   kPrefetchAtStart:    as soon as the compute waves hold the current unit's state in
//                        registers (one more barrier), so that the state read overlaps the
//                        conv phase as well. Measured faster up to 4 GiB of snapshots per call
//                        and slower beyond (the dispatch rule below).
// Loading it any later, in front of a token's snapshot stores, measured 4-20 % slower.
enum StatePrefetch { kPrefetchAfterConv = 1, kPrefetchAtStart = 2 };

// A unit as the producer hands it over: its index (lb < 0: no more units), pool rows,
// whether its rows are inside the pools (a padding unit is skipped whole), and whether it
// was the last of its q/k group to count in.
struct UnitDesc {
  int lb, cs_row, st_row, in_row, last, valid;
};

template <class CF, typename R>
struct alignas(16) StreamSmem {
  Smem<CF, R> s;                // the staged inputs (written by the producer) and the unit's rows
  f32x4 st[CF::K * CF::V / 4];  // the next unit's state tile, K rows of V floats as in HBM
  float alog;                   // A_log of the next unit's value head
  UnitDesc desc[2];             // the unit handed over at the last barrier, by parity
};

typedef __attribute__((address_space(3))) void lds_void_t;
typedef const __attribute__((address_space(1))) void global_void_t;

// LDS-direct load: every active lane reads BYTES at src, and the wave writes lane i's
// value to lds + 16 i (16-byte loads) or lds + 4 i (4- and 2-byte loads, zero-extended).
// The LDS address must be the same for every lane. NT: the streaming hint.
// The LDS pointer is taken from the generic address's low 32 bits (the offset within the
// workgroup's LDS) rather than by an address-space cast: the cast carries a null check,
// and where the compiler merges those checks across branches of the producer it emits an
// instruction that reads the shared-memory aperture register as an operand the gfx950
// encoding does not allow, and the build fails.
template <int BYTES, bool NT = false>
__device__ __forceinline__ void lds_direct(const void* src, void* lds_generic) {
  lds_void_t* lds = (lds_void_t*)(uintptr_t)(uint32_t)(uintptr_t)lds_generic;
  if constexpr (BYTES == 16 && NT)
    __builtin_amdgcn_global_load_lds((global_void_t*)src, lds, 16, 0, 2);
  else if constexpr (BYTES == 16)
    __builtin_amdgcn_global_load_lds((global_void_t*)src, lds, 16, 0, 0);
  else if constexpr (BYTES == 4)
    __builtin_amdgcn_global_load_lds((global_void_t*)src, lds, 4, 0, 0);
  else
    __builtin_amdgcn_global_load_lds((global_void_t*)src, lds, 2, 0, 0);
}

// The producer's side of the compute waves' barriers. A plain barrier, with no wait, so
// that the producer's loads stay in flight across it; the memory clobber keeps the
// compiler from moving the loads across it.
__device__ __forceinline__ void producer_barrier() { asm volatile("s_barrier" ::: "memory"); }
// The hand-over barrier: every load of the producer has landed in LDS and its unit
// descriptor is written before the compute waves pass it.
__device__ __forceinline__ void producer_handover() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Producer: the pool rows of unit lb (lb < 0: no unit).
template <class CF>
__device__ __forceinline__ UnitDesc stream_rows(const Args& a, const int lb) {
  UnitDesc d;
  d.lb = lb;
  d.last = 1;
  d.cs_row = d.st_row = d.in_row = 0;
  d.valid = 0;
  if (lb < 0) return d;
  const int n = (lb / CF::NVT) / a.HV;
  d.cs_row = a.cs_idx ? a.cs_idx[n] : n;
  d.st_row = a.st_idx ? a.st_idx[n] : n;
  d.in_row = a.in_idx ? a.in_idx[n] : n;
  d.valid = !(d.cs_row < 0 || d.cs_row >= a.cs_slots || d.st_row < 0 || d.st_row >= a.st_slots || d.in_row < 0 ||
              d.in_row >= a.in_slots);
  return d;
}

// Producer: issue the LDS-direct loads of a valid unit's small inputs into the staging
// record, each block of 16-byte vectors in the order the grid and queue units stage them
// (the same LDS layout), 64 vectors per instruction. Not waited for here.
template <class CF, typename R>
__device__ __forceinline__ void stream_stage_inputs(const Args& a, StreamSmem<CF, R>& ss, const UnitDesc& d,
                                                    const int lane) {
  constexpr int K = CF::K, NCH = CF::NCH, E16 = CF::E16;
  const int T = a.T, H = a.H, HV = a.HV, C = a.C;
  const int vt = d.lb % CF::NVT;
  const int unit = d.lb / CF::NVT;
  const int hv = unit % HV, n = unit / HV;
  const int h = hv / a.g;
  Smem<CF, R>& s = ss.s;
  const R* xq = static_cast<const R*>(a.mixed_qkv);
  const R* wq = static_cast<const R*>(a.conv_weight);
  const R* cq = static_cast<const R*>(a.conv_state);
  const R* gq = static_cast<const R*>(a.gate);
  const R* bq = static_cast<const R*>(a.beta);
  const int PA = NCH / E16;
  const int nA = T * PA;  // new tokens
  for (int k = 0; k * 64 < nA; ++k) {
    const int ci = k * 64 + lane;
    if (ci < nA) {
      const int t = ci / PA, pe = (ci - t * PA) * E16;
      lds_direct<16>(xq + (size_t)(n * T + t) * C + gchan<CF>(pe, h, H, hv, vt),
                     reinterpret_cast<char*>(s.xs) + k * 1024);
    }
  }
  constexpr int nB = 3 * NCH / E16;  // conv cache
#pragma unroll
  for (int k = 0; k * 64 < nB; ++k) {
    const int ci = k * 64 + lane;
    if (ci < nB) {
      const int e = ci * E16, lc = e / 3;
      lds_direct<16>(cq + ((size_t)d.cs_row * C + gchan<CF>(lc, h, H, hv, vt)) * 3 + (e - lc * 3),
                     reinterpret_cast<char*>(s.cs) + k * 1024);
    }
  }
  constexpr int nC = 4 * NCH / E16;  // conv taps
#pragma unroll
  for (int k = 0; k * 64 < nC; ++k) {
    const int ci = k * 64 + lane;
    if (ci < nC) {
      const int e = ci * E16, lc = e / 4;
      lds_direct<16>(wq + (size_t)gchan<CF>(lc, h, H, hv, vt) * 4 + (e - lc * 4),
                     reinterpret_cast<char*>(s.ws) + k * 1024);
    }
  }
  const int nD = T * K / E16;  // gate
  for (int k = 0; k * 64 < nD; ++k) {
    const int ci = k * 64 + lane;
    if (ci < nD) {
      const int e = ci * E16, t = e / K;
      lds_direct<16>(gq + ((size_t)(n * T + t) * HV + hv) * K + (e - t * K), reinterpret_cast<char*>(s.gs) + k * 1024);
    }
  }
  constexpr int nE = K / 4;  // dt_bias (fp32)
#pragma unroll
  for (int k = 0; k * 64 < nE; ++k) {
    const int ci = k * 64 + lane;
    if (ci < nE) lds_direct<16>(a.dt_bias + (size_t)hv * K + ci * 4, reinterpret_cast<char*>(s.dtb) + k * 1024);
  }
  if (lane < T) lds_direct<(int)sizeof(R)>(bq + (size_t)(n * T + lane) * HV + hv, s.bs);
  if (lane == 0) lds_direct<4>(a.A_log + hv, &ss.alog);
}

// Producer: issue the LDS-direct loads of a valid unit's state tile, 1 KiB per
// instruction, with the streaming hint: instructions [j0, j1) of its 64. Not waited for
// here.
template <class CF, typename R>
__device__ __forceinline__ void stream_stage_state(const Args& a, StreamSmem<CF, R>& ss, const UnitDesc& d,
                                                   const int lane, const int j0 = 0, const int j1 = CF::K * CF::V / 256) {
  constexpr int K = CF::K, V = CF::V;
  const int hv = (d.lb / CF::NVT) % a.HV;
  const float* sp = a.state + ((size_t)d.st_row * a.HV + hv) * ((size_t)K * V) + lane * 4;
#pragma unroll
  for (int j = j0; j < j1; ++j)
    lds_direct<16, true>(sp + j * 256, reinterpret_cast<char*>(ss.st) + j * 1024);
}

// Producer: count unit d into its q/k group once its reads have landed (the caller has
// waited for them), as a grid or queue unit counts itself in after its staged loads;
// returns whether it was the last of the group, which then writes the rolled q/k cache.
__device__ __forceinline__ int stream_count_in(const Args& a, const UnitDesc& d, const int nvt, const int lane) {
  if (!d.valid || a.group <= 1) return 1;
  const int unit = d.lb / nvt;
  const int hv = unit % a.HV, n = unit / a.HV, h = hv / a.g;
  uint32_t* c = a.counters + (size_t)n * a.H + h;
  uint32_t prev = 0;
  if (lane == 0) prev = __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  prev = (uint32_t)__builtin_amdgcn_readfirstlane((int)prev);
  const int last = prev == (uint32_t)(a.group - 1);
  if (last && lane == 0) __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return last;
}

// The producer wave. It passes exactly the barriers the compute waves pass for each unit
// (B0 with kPrefetchAtStart, B1, B2, one per token, then the hand-over; a padding unit only
// the hand-over), decided by the same descriptor and T.
template <class CF, typename R>
__device__ __forceinline__ void stream_producer(const Args& a, StreamSmem<CF, R>& ss, const int units, const int G) {
  const int lane = threadIdx.x & 63;
  uint32_t* qc = a.counters + (size_t)a.N * a.H;  // ticket, then leave count
  UnitDesc d = stream_rows<CF>(a, xcd_order(blockIdx.x, G));
  if (d.valid) {
    stream_stage_inputs<CF, R>(a, ss, d, lane);
    stream_stage_state<CF, R>(a, ss, d, lane);
  }
  uint32_t tk = 0;
  if (lane == 0) tk = __hip_atomic_fetch_add(qc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  tk = (uint32_t)__builtin_amdgcn_readfirstlane((int)tk);
  if (lane == 0) ss.desc[0] = d;
  UnitDesc nd = stream_rows<CF>(a, kda_queue_unit(tk, units, G));  // the unit after it
  producer_handover();
  // The first unit is counted into its q/k group after the hand-over (its loads have
  // landed): the atomic flies while the compute waves copy the state and run the conv, and
  // its result reaches the descriptor before B1, where the compute waves first read it
  // (measured on MI355X: 0.2-0.9 % faster on shared q/k heads, neutral elsewhere).
  // Later units are counted in at the last token of the unit before them, below.
  const bool count0 = d.valid && a.group > 1;
  uint32_t* c0 = a.counters + (size_t)((d.lb / CF::NVT) / a.HV) * a.H + ((d.lb / CF::NVT) % a.HV) / a.g;
  uint32_t prev0 = 0;
  if (count0 && lane == 0) prev0 = __hip_atomic_fetch_add(c0, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int it = 0;; ++it) {
    const UnitDesc cur = ss.desc[it & 1];
    if (cur.lb < 0) break;
    const bool drew = nd.lb >= 0;
    const bool state_at_start = a.prefetch == kPrefetchAtStart && cur.valid;
    // With the state loaded at the start, half of the next tile is issued at B0 and half
    // after B1: the counter holds at most 63 loads, so issuing all 64 at B0 stalled the
    // producer on the first one's return and could make it late for B1 (measured on
    // MI355X: 0.2-1.1 % faster on seven of eight shapes, large_batch at T = 2 by 1.1 %;
    // 48 or 56 first gained less, 16 first lost).
    if (state_at_start) {
      producer_barrier();  // B0: the compute waves hold the state tile in registers
      if (nd.valid) stream_stage_state<CF, R>(a, ss, nd, lane, 0, 32);
    }
    if (it == 0 && count0) {
      prev0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)prev0);
      const int last0 = prev0 == (uint32_t)(a.group - 1);
      if (last0 && lane == 0) __hip_atomic_store(c0, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (lane == 0) ss.desc[0].last = last0;
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
    if (cur.valid) producer_barrier();  // B1: the compute waves are done with the staged inputs
    const bool stage = drew && nd.valid;
    if (stage) {
      if (state_at_start) {
        stream_stage_state<CF, R>(a, ss, nd, lane, 32, CF::K * CF::V / 256);  // the rest
      } else {
        stream_stage_inputs<CF, R>(a, ss, nd, lane);
        stream_stage_state<CF, R>(a, ss, nd, lane, 0, 32);
      }
    }
    // after B2 (or at once for a padding unit): the inputs (state at the start) or the
    // second half of the state tile (state after the conv). Issued together after B1,
    // these loads outran the 63 the counter holds, and the producer came late to B2
    // (measured on MI355X: large_batch 414.6 -> 410.5 us, gva 92.3 -> 91.2 us; within
    // 0.3 % either way on the shapes it did not help).
    auto stage_late = [&]() {
      if (stage) {
        if (state_at_start)
          stream_stage_inputs<CF, R>(a, ss, nd, lane);
        else
          stream_stage_state<CF, R>(a, ss, nd, lane, 32, CF::K * CF::V / 256);
      }
    };
    if (!cur.valid) stage_late();
    // The ticket for the unit after nd is drawn at the last token's barrier, not here: near
    // the end of the queue a unit drawn early waits in a workgroup that still has most of
    // the current unit to run while others fall idle. At that barrier the producer also
    // counts nd into its q/k group (its loads landed long before) and reads the new unit's
    // pool rows, so the last token's update and stores cover all three round trips and the
    // hand-over only writes the descriptor (measured on MI355X: the late draw 0.3-1.1 %
    // faster on eight shapes, large_batch 417.1 -> 414.2 us; the count-in moved with it
    // another 0.3-0.9 % on shared q/k heads, gva 93.9 -> 93.1 us).
    UnitDesc nn;  // the unit after nd
    auto draw_and_count = [&]() {
      if (drew) {
        if (lane == 0) tk = __hip_atomic_fetch_add(qc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        asm volatile("s_waitcnt vmcnt(1)" ::: "memory");  // nd's loads have landed; the ticket may fly
        nd.last = stream_count_in(a, nd, CF::NVT, lane);
        tk = (uint32_t)__builtin_amdgcn_readfirstlane((int)tk);
        nn = stream_rows<CF>(a, kda_queue_unit(tk, units, G));
      } else {
        nn = stream_rows<CF>(a, -1);
      }
    };
    if (cur.valid) {
      producer_barrier();  // B2
      stage_late();
      for (int t = 0; t < a.T; ++t) {
        producer_barrier();  // one per token
        if (t == a.T - 1) draw_and_count();
      }
    } else {
      draw_and_count();
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (lane == 0) ss.desc[(it + 1) & 1] = nd;
    nd = nn;
    producer_handover();
  }
  // every ticket this workgroup drew has been seen (the last one past the end): count out;
  // the last workgroup to leave zeroes the ticket and leave counts for the next call
  if (lane == 0) {
    const uint32_t left = __hip_atomic_fetch_add(qc + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (left == (uint32_t)G - 1) {
      __hip_atomic_store(qc, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(qc + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// The compute waves' part of one unit the producer staged: the same phases and barriers
// as a queue unit, from LDS.
template <class CF, typename R>
__device__ __forceinline__ void stream_unit(const Args& a, StreamSmem<CF, R>& ss, const UnitDesc& d, const int slot) {
  constexpr int V = CF::V, RPL = CF::RPL, Q = CF::Q, LPR = CF::LPR;
  Smem<CF, R>& s = ss.s;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int vt = d.lb % CF::NVT;
  const int unit = d.lb / CF::NVT;
  const int hv = unit % a.HV, n = unit / a.HV;
  const int h = hv / a.g;
  const int grp = wave / CF::NW, wv = wave - grp * CF::NW;
  const int c4 = lane % LPR, qq = lane / LPR;
  const int col = vt * CF::WT + grp * CF::VT + c4 * 4;
  const int row0 = wv * CF::RW + qq;
  f32x4 S[RPL];
#pragma unroll
  for (int r = 0; r < RPL; ++r) S[r] = ss.st[((row0 + r * Q) * V + col) / 4];
  const float alog = ss.alog;
  if (a.prefetch == kPrefetchAtStart) __syncthreads();  // B0: the producer may load the next state tile
  const bool qk_owner = (hv % a.g == 0) && vt == 0;
  conv_and_gates<CF, R>(a, s, qk_owner, alog);
  __syncthreads();  // B1
  l2norm_tokens<CF, R>(a, s);
  if (tid == 0) s.last = ss.desc[slot].last;  // set by B1 (the first unit's only just before it)
  __syncthreads();  // B2
  token_loop<CF, R, true>(a, s, S, UnitAt{n, hv, h, vt, d.cs_row, d.in_row}, qk_owner);
}

// Whole-V workgroups of CF::NTHR compute threads plus the producer wave, one per CU (the
// LDS record alone holds a CU), grid = resident workgroups (<= units).
template <class CF, typename R>
__global__ __launch_bounds__(CF::NTHR + 64) void kda_verify_stream_kernel(const Args a) {
  __shared__ StreamSmem<CF, R> ss;
  const int units = a.N * a.HV * CF::NVT;
  const int G = gridDim.x;
  if ((int)threadIdx.x >= CF::NTHR) {
    stream_producer<CF, R>(a, ss, units, G);
    return;
  }
  __syncthreads();  // the first unit is in LDS
  for (int it = 0;; ++it) {
    const UnitDesc d = ss.desc[it & 1];
    if (d.lb < 0) break;
    if (d.valid) stream_unit<CF, R>(a, ss, d, it & 1);
    __syncthreads();  // hand-over: the producer has staged the next unit
  }
}

// Whether the stream schedule's LDS record of CF fits a CU (160 KiB).
template <class CF, typename R>
constexpr bool stream_fits() {
  return CF::K == 128 && CF::WT == CF::V && CF::G == 1 && !CF::PRE && sizeof(StreamSmem<CF, R>) <= 160 * 1024;
}

// Unfused form, first kernel: width-4 causal conv + SiLU for every channel, one thread per
// (sequence, channel) walking the T tokens with a 3-value raw window; writes the fp32
// activations to act [N,T,C], the per-token raw windows and the rolled cache.
struct ConvArgs {
  const void* x;
  const void* w;
  void* conv_state;
  void* conv_window;
  void* act;
  const int32_t* cs_idx;
  const int32_t* st_idx;
  const int32_t* in_idx;
  int cs_slots, st_slots, in_slots;
  int N, T, C;
};

template <typename R>
__global__ __launch_bounds__(256) void kda_conv_silu_kernel(const ConvArgs a) {
  const int n = blockIdx.y, c = blockIdx.x * 256 + threadIdx.x;
  if (c >= a.C) return;
  const int cs_row = a.cs_idx ? a.cs_idx[n] : n;
  const int st_row = a.st_idx ? a.st_idx[n] : n;
  const int in_row = a.in_idx ? a.in_idx[n] : n;
  if (cs_row < 0 || cs_row >= a.cs_slots || st_row < 0 || st_row >= a.st_slots || in_row < 0 ||
      in_row >= a.in_slots)
    return;
  const R* x = static_cast<const R*>(a.x);
  const R* w = static_cast<const R*>(a.w) + (size_t)c * 4;
  R* cs = static_cast<R*>(a.conv_state) + ((size_t)cs_row * a.C + c) * 3;
  R* cw = static_cast<R*>(a.conv_window);
  float* act = static_cast<float*>(a.act);
  const float w0 = up(w[0]), w1 = up(w[1]), w2 = up(w[2]), w3 = up(w[3]);
  R e0 = cs[0], e1 = cs[1], e2 = cs[2];
  for (int t = 0; t < a.T; ++t) {
    const R e3 = x[((size_t)n * a.T + t) * a.C + c];
    const float y = fmaf(w3, up(e3), fmaf(w2, up(e2), fmaf(w1, up(e1), w0 * up(e0))));
    act[((size_t)n * a.T + t) * a.C + c] = silu_fast(y);
    R* wrow = cw + (((size_t)in_row * a.T + t) * a.C + c) * 3;
    wrow[0] = e1;
    wrow[1] = e2;
    wrow[2] = e3;
    e0 = e1;
    e1 = e2;
    e2 = e3;
  }
  cs[0] = e0;
  cs[1] = e1;
  cs[2] = e2;
}

// Accept step: one WG per (sequence, value head) copies the state snapshot of the last
// accepted token into the state pool, and one slice of that token's raw conv window into
// the conv cache pool (the HV WGs of a sequence split the row between them). Pure 16-byte
// copies.
struct CommitArgs {
  const int32_t* accepted;
  const float* inter_ssm;
  const void* conv_window;
  float* state;
  void* conv_state;
  const int32_t* cs_idx;
  const int32_t* st_idx;
  const int32_t* in_idx;
  int cs_slots, st_slots, in_slots;
  int N, T, HV, C;
  int kv4;     // K * V / 4 vectors per unit
  int cs_vec;  // 16-byte vectors in one conv cache row (C * 3 elements)
};

// NT threads, U vectors per thread in each round, all loads of a round in flight before
// its stores, which carry the streaming hint; the WG's slice of the conv row rides with the
// first round. Two shapes, picked by the number of units in kda_verify_commit.
template <int NT, int U>
__global__ __launch_bounds__(NT) void kda_commit_kernel(const CommitArgs a) {
  const int unit = xcd_order(blockIdx.x, gridDim.x), n = unit / a.HV, hv = unit % a.HV;
  const int acc = a.accepted[n];
  const int cs_row = a.cs_idx ? a.cs_idx[n] : n;
  const int st_row = a.st_idx ? a.st_idx[n] : n;
  const int in_row = a.in_idx ? a.in_idx[n] : n;
  if (acc < 1 || acc > a.T || cs_row < 0 || cs_row >= a.cs_slots || st_row < 0 || st_row >= a.st_slots ||
      in_row < 0 || in_row >= a.in_slots)
    return;
  const int tid = threadIdx.x;
  const size_t src_tok = (size_t)in_row * a.T + (acc - 1);
  const f32x4* __restrict__ src = reinterpret_cast<const f32x4*>(a.inter_ssm) + (src_tok * a.HV + hv) * (size_t)a.kv4;
  f32x4* __restrict__ dst = reinterpret_cast<f32x4*>(a.state) + ((size_t)st_row * a.HV + hv) * (size_t)a.kv4;
  const u32x4* __restrict__ cw = reinterpret_cast<const u32x4*>(a.conv_window) + src_tok * (size_t)a.cs_vec;
  u32x4* __restrict__ cs = reinterpret_cast<u32x4*>(a.conv_state) + (size_t)cs_row * a.cs_vec;
  // this WG's vectors [c0, c1) of the conv row
  const int per = (a.cs_vec + a.HV - 1) / a.HV;
  const int c0 = min(a.cs_vec, hv * per), c1 = min(a.cs_vec, c0 + per);
  for (int base = 0; base < a.kv4; base += U * NT) {
    f32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base + u * NT + tid;
      if (i < a.kv4) v[u] = __builtin_nontemporal_load(src + i);
    }
    const bool hc = base == 0 && c0 + tid < c1;
    u32x4 c;
    if (hc) c = cw[c0 + tid];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base + u * NT + tid;
      if (i < a.kv4) store_snapshot<kStoreNT>(reinterpret_cast<float*>(dst + i), v[u]);
    }
    if (hc) cs[c0 + tid] = c;
  }
  for (int i = c0 + NT + tid; i < c1; i += NT) cs[i] = cw[i];
}

__global__ void zero_words(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// ----------------------------------------------------------------------------------
// host side
// ----------------------------------------------------------------------------------
// A launch configuration: tile width, snapshot store policy, workgroups-per-CU cap,
// column groups and schedule.
struct Tile {
  int vt;              // V columns per WG
  int stp;             // StorePolicy
  int occ = 0;         // workgroups per CU cap (lds_reservation), 0 = none
  int g = 1;           // column groups of 4 waves sharing the WG's staging and conv
  bool queue = false;   // resident workgroups pulling units from a counter (whole-V only)
  int order = kOrderXcdRanges;  // UnitOrder of the grid
  bool stream = false;  // the queue with a producer wave (whole-V, one group, T <= 8)
  int prefetch = kPrefetchAfterConv;  // StatePrefetch of the stream schedule
};
using LaunchFn = hipError_t (*)(const Args&, const Tile&, hipStream_t);

// LDS a workgroup reserves so that at most `wg_per_cu` of them share a CU (0: no cap
// beyond the kernel's own LDS and VGPRs). The reservation is dynamic LDS on top of the
// kernel's static record; the kernel never touches it. Sizes from MI355X measurements
// (rocprofv3 MeanOccupancyPerCU and timings): workgroups holding 98 KiB run one per CU,
// 53 KiB two, 35.5 KiB four, 23.5 KiB six.
size_t lds_reservation(int wg_per_cu) {
  switch (wg_per_cu) {
    case 1: return 100352;
    case 2: return 54272;
    case 4: return 36352;
    case 6: return 24064;
    default: return 0;
  }
}

// Workgroups of kernel `fn` that can be resident on the current device at once: the
// compute units times the per-CU cap, or times the occupancy the runtime computes for
// the kernel when there is no cap. 0 when the runtime cannot tell.
long long resident_workgroups(const void* fn, int threads, size_t dyn_lds, int wg_per_cu) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cu_count[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int cus = cu_count[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      return 0;
    cu_count[dev].store(cus, std::memory_order_relaxed);
  }
  int per_cu = wg_per_cu;
  if (per_cu == 0 && (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, dyn_lds) != hipSuccess ||
                      per_cu <= 0))
    return 0;
  return (long long)cus * per_cu;
}

template <class CF, typename R>
hipError_t launch(const Args& a, const Tile& tl, hipStream_t stream) {
  const long long units = (long long)a.N * a.HV * CF::NVT;
  Args copy = a;
  copy.group = a.g * CF::NVT;
  copy.order = tl.order;
  copy.prefetch = tl.prefetch;
  void* args[] = {&copy};
  const size_t want = lds_reservation(tl.occ), have = sizeof(Smem<CF, R>);
  const size_t dyn = want > have ? want - have : 0;
  if (tl.stream) {
    if constexpr (stream_fits<CF, R>()) {
      const void* fn = reinterpret_cast<const void*>(&kda_verify_stream_kernel<CF, R>);
      const long long slots = resident_workgroups(fn, CF::NTHR + 64, 0, 1);
      if (slots <= 0) return hipErrorInvalidConfiguration;
      return hipLaunchKernel(fn, dim3((unsigned)(units < slots ? units : slots)), dim3(CF::NTHR + 64), args, 0,
                             stream);
    } else {
      return hipErrorInvalidConfiguration;  // whole-V, one group, T <= 8 only (check_params)
    }
  }
  if (tl.queue) {
    if constexpr (CF::WT == CF::V && !CF::PRE) {
      const void* fn = reinterpret_cast<const void*>(&kda_verify_queue_kernel<CF, R>);
      const long long slots = resident_workgroups(fn, CF::NTHR, dyn, tl.occ);
      if (slots <= 0) return hipErrorInvalidConfiguration;
      return hipLaunchKernel(fn, dim3((unsigned)(units < slots ? units : slots)), dim3(CF::NTHR), args, dyn, stream);
    } else {
      return hipErrorInvalidConfiguration;  // whole-V fused workgroups only (check_params)
    }
  }
  return hipLaunchKernel(reinterpret_cast<const void*>(&kda_verify_kernel<CF, R>), dim3((unsigned)units),
                         dim3(CF::NTHR), args, dyn, stream);
}

// AUTO launch for K = V = 128, from two dispatch sweeps on MI355X (bench.py --sweep, two
// boxes: 486 shapes with H = 8-64 and 399 with H = 12, 24, 48, one or two value heads per
// q/k head, T = 1-8, 128-4096 (sequence, value head) units; 27 launches each, timed
// round-robin over rotated buffer sets). Five buckets:
//   1. <= 64 units (<= 128 at T = 2): the 32-column split, four workgroups per unit, so that
//      a launch-latency-bound call spreads over more CUs;
//   2. <= 512 units, one generation of whole-V workgroups (all resident at once, no cap):
//      four column groups up to 128 units and at T = 1 up to 256 (a 16-wave workgroup runs
//      one per CU, so 256 of them are one generation); one group at T = 1 beyond that, from
//      448 units, and at odd T from 256 units; two groups otherwise. Streaming stores
//      (policy 1) at T = 2 and 4 and with four groups, device scope (policy 2) otherwise;
//   3. < 1024 units, or < 1280 units at T = 2, or < 3072 at T = 1: the uncapped whole-V grid;
//   4. < 1280 units at T = 3, 4: two whole-V workgroups per CU;
//   5. otherwise the stream schedule (the queue above T = 8): the next unit's state loaded
//      at the start of the current one up to 65536 snapshot tiles of 64 KiB (4 GiB) per
//      call, after its conv beyond. On a third sweep (240 shapes of 1024-8192 units, T = 2-8,
//      with both stream launches) the stream was the fastest launch on 169 shapes and the
//      queue it replaced 4-7 % slower on average at T = 2-4; A/B runs on 40 shapes up to
//      32768 units set the 4 GiB point (beyond it the later load was 0.3-3 % ahead); at T = 1
//      a sweep of 70 shapes put the stream ahead of the grid from 3072 units (by 1-15 %, 88 %
//      of the HBM peak at 32768 units) and behind it up to 2048. Once the stream's producer
//      issued its loads spread over the unit's barriers and took its tickets at the last
//      token, the sweeps, re-run, put the stream ahead at T = 2-4 from 1344 units, the first
//      size above 1024 they hold (by 2.9-7.3 % on average per T and size), behind at 1024 (by
//      3-10 %), and the grid still ahead at T = 1 up to 2048; buckets 3 and 4 now end at 1280
//      units for T = 2-4, between those two sizes.
// Buckets 3-5 store at device scope. The unit order follows from the launch (choose_tile):
// pairs for uncapped whole-V grids. Every launch uses the same K split (32 rows per wave)
// and partial-sum tree, so all return bit-identical results; cap, schedule and order only
// change which CU runs a unit, and when.
Tile auto_tile_128(long long units, int T) {
  if (units <= 64 || (units <= 128 && T == 2)) return Tile{32, kStoreNT};
  if (units <= 512) {
    int g;
    if (units <= 128 || (T == 1 && units <= 256))
      g = 4;
    else if (T == 1 || units >= 448 || (T % 2 == 1 && units >= 256))
      g = 1;
    else
      g = 2;
    return Tile{128, (T == 2 || T == 4 || g == 4) ? kStoreNT : kStoreNTDev, 0, g};
  }
  if (units < 1024 || (units < 1280 && T == 2) || (units < 3072 && T == 1)) return Tile{128, kStoreNTDev};
  if (units < 1280 && T <= 4) return Tile{128, kStoreNTDev, 2};
  if (T > 8) return Tile{128, kStoreNTDev, 1, 1, true};
  Tile t{128, kStoreNTDev, 1, 1};
  t.stream = true;
  t.prefetch = units * T <= 65536 ? kPrefetchAtStart : kPrefetchAfterConv;
  return t;
}

// The AUTO choice with the caller's overrides applied. A cap belongs to the AUTO tile: when
// the tile is chosen by the caller (tile_columns or an explicit variant), the AUTO cap is
// not applied and only max_wg_per_cu sets one.
Tile choose_tile(const kda_verify_params* p) {
  const int K = p->K, V = p->V;
  const bool caller_tile = p->tile_columns != 0 || p->variant != KDA_VARIANT_AUTO;
  Tile t;
  if (K == 128 && V == 128) {
    t = auto_tile_128((long long)p->N * p->HV, p->T);
    if (caller_tile) {
      t.occ = 0;
      t.g = 1;
      t.queue = false;
      t.stream = false;
    }
    if (p->tile_columns != 0)
      t.vt = p->tile_columns;
    else if (p->variant == KDA_VARIANT_LARGE)
      t.vt = 128;
    else if (p->variant == KDA_VARIANT_SMALL)
      t.vt = 32;
    else if (p->schedule >= 2 || p->column_groups > 1)
      t.vt = 128;  // the queue, the stream and column groups run whole-V workgroups
    if (p->store_policy != 0) t.stp = p->store_policy == 2 ? kStoreNTDev : kStoreNT;
    // fp32 inputs at T > 8: a whole-V workgroup's staged inputs and conv windows would not
    // fit in LDS; two 64-column workgroups give the same bits
    if (p->in_dtype == KDA_F32 && p->T > 8 && t.vt == 128) {
      t.vt = 64;
      t.g = 1;
      t.queue = false;
      t.stream = false;
    }
  } else {
    t = K == 64 && V == 64 ? Tile{p->variant == KDA_VARIANT_SMALL ? 32 : 64, kStoreNT} : Tile{16, kStoreNT};
  }
  if (p->max_wg_per_cu != 0) t.occ = p->max_wg_per_cu == 8 ? 0 : p->max_wg_per_cu;
  if (p->column_groups != 0) t.g = p->column_groups;
  if (p->schedule != 0) {
    t.queue = p->schedule == 2;
    t.stream = p->schedule == 3;
  }
  // the stream runs one whole-V group per CU: a caller's column groups or cap take the AUTO
  // stream back to the queue, which honours them
  if (t.stream && p->schedule != 3 && (t.g > 1 || t.occ != 1)) {
    t.stream = false;
    t.queue = true;
  }
  if (t.stream) {  // one whole-V workgroup (one group) per CU, held there by its LDS
    t.g = 1;
    t.occ = 1;
    if (p->prefetch != 0) t.prefetch = p->prefetch;
  }
  // unit order of the grid: pairs when whole-V workgroups run without a cap (every
  // workgroup resident at once), XCD ranges otherwise
  if (p->unit_order != 0)
    t.order = p->unit_order;
  else
    t.order = t.vt == V && t.occ == 0 && !t.queue ? kOrderPairs : kOrderXcdRanges;
  return t;
}

template <typename R, int TMAX, int PRE>
LaunchFn pick_tmax(int K, int V, Tile tl) {
  if (K == 128 && V == 128) {
    // whole-V tiles of fp32 inputs at T > 8 would exceed the LDS of a CU (choose_tile
    // never asks for them)
    constexpr bool whole_v = !(sizeof(R) == 4 && TMAX > 8 && PRE == 0);
    if constexpr (whole_v) {
      if (tl.vt == 128 && tl.g == 4)
        return tl.stp == kStoreNTDev ? &launch<Cfg<R, 128, 128, 32, 4, TMAX, kStoreNTDev, PRE, 4>, R>
                                   : &launch<Cfg<R, 128, 128, 32, 4, TMAX, kStoreNT, PRE, 4>, R>;
      if (tl.vt == 128 && tl.g == 2)
        return tl.stp == kStoreNTDev ? &launch<Cfg<R, 128, 128, 64, 4, TMAX, kStoreNTDev, PRE, 2>, R>
                                   : &launch<Cfg<R, 128, 128, 64, 4, TMAX, kStoreNT, PRE, 2>, R>;
      if (tl.vt == 128)
        return tl.stp == kStoreNTDev ? &launch<Cfg<R, 128, 128, 128, 4, TMAX, kStoreNTDev, PRE>, R>
                                   : &launch<Cfg<R, 128, 128, 128, 4, TMAX, kStoreNT, PRE>, R>;
    } else {
      if (tl.vt == 128) return nullptr;
    }
    if (tl.g != 1) return nullptr;
    if (tl.vt == 64)
      return tl.stp == kStoreNTDev ? &launch<Cfg<R, 128, 128, 64, 4, TMAX, kStoreNTDev, PRE>, R>
                                 : &launch<Cfg<R, 128, 128, 64, 4, TMAX, kStoreNT, PRE>, R>;
    return tl.stp == kStoreNTDev ? &launch<Cfg<R, 128, 128, 32, 4, TMAX, kStoreNTDev, PRE>, R>
                               : &launch<Cfg<R, 128, 128, 32, 4, TMAX, kStoreNT, PRE>, R>;
  }
  if (K == 64 && V == 64) {
    if (tl.vt == 64) return &launch<Cfg<R, 64, 64, 64, 2, TMAX, kStoreNT, PRE>, R>;
    return &launch<Cfg<R, 64, 64, 32, 2, TMAX, kStoreNT, PRE>, R>;
  }
  if (K == 16 && V == 16) return &launch<Cfg<R, 16, 16, 16, 1, TMAX, kStoreNT, PRE>, R>;
  return nullptr;
}

template <typename R, int PRE>
LaunchFn pick(int K, int V, Tile tl, int T) {
  if (T <= 4) return pick_tmax<R, 4, PRE>(K, V, tl);
  if (T <= 8) return pick_tmax<R, 8, PRE>(K, V, tl);
  return pick_tmax<R, 16, PRE>(K, V, tl);
}

LaunchFn pick_launch(const kda_verify_params* p, Tile tl, bool pre) {
  if (p->in_dtype == KDA_BF16)
    return pre ? pick<uint16_t, 1>(p->K, p->V, tl, p->T) : pick<uint16_t, 0>(p->K, p->V, tl, p->T);
  return pre ? pick<uint32_t, 1>(p->K, p->V, tl, p->T) : pick<uint32_t, 0>(p->K, p->V, tl, p->T);
}

// Device address of this GPU's copy of `scratch`, looked up once per device with that
// device current and kept for later calls.
hipError_t scratch_on_current_device(uint32_t** out) {
  constexpr int kMaxDevices = 64;
  struct Slot {
    std::once_flag once;
    hipError_t err = hipSuccess;
    uint32_t* ptr = nullptr;
  };
  static Slot slots[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  Slot& sl = slots[dev];
  std::call_once(sl.once, [&sl] {
    void* ptr = nullptr;
    sl.err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    sl.ptr = static_cast<uint32_t*>(ptr);
  });
  if (sl.err != hipSuccess) return sl.err;
  if (!sl.ptr) return hipErrorInvalidSymbol;
  *out = sl.ptr;
  return hipSuccess;
}

// Zero `words` counters on `stream` with the fill kernel (never a memset node).
hipError_t launch_zero_words(uint32_t* p, size_t words, hipStream_t stream) {
  size_t blocks = (words + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  if (blocks == 0) return hipSuccess;
  void* args[] = {&p, &words};
  return hipLaunchKernel(reinterpret_cast<const void*>(&zero_words), dim3((unsigned)blocks), dim3(256), args, 0,
                         stream);
}

bool supported_kv(int K, int V) { return K == V && (K == 16 || K == 64 || K == 128); }

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

struct Range {
  uintptr_t lo, hi;
};
bool overlap(Range x, Range y) { return x.lo < y.hi && y.lo < x.hi; }

}  // namespace kda

using namespace kda;

extern "C" {

void kda_verify_params_init(kda_verify_params* p, int32_t N, int32_t T, int32_t H, int32_t HV, int32_t K,
                            int32_t V) {
  if (!p) return;
  memset(p, 0, sizeof(*p));
  p->N = N;
  p->T = T;
  p->H = H;
  p->HV = HV;
  p->K = K;
  p->V = V;
  p->in_dtype = KDA_BF16;
  p->gate_mode = KDA_GATE_SOFTPLUS;
  p->variant = KDA_VARIANT_AUTO;
  p->lower_bound = -5.0f;
  p->softplus_beta = 1.0f;
  p->softplus_threshold = 20.0f;
  p->scale = 0.0f;
  p->l2norm_eps = 1e-6f;
  p->tile_columns = 0;
  p->store_policy = 0;
  p->max_wg_per_cu = 0;
  p->column_groups = 0;
  p->schedule = 0;
  p->unit_order = 0;
  p->prefetch = 0;
}

static kda_status check_params(const kda_verify_params* p) {
  if (!p) return KDA_ERR_NULL;
  if (p->N < 0 || p->T < 1 || p->T > KDA_MAX_T || p->H < 1 || p->HV < p->H || p->HV % p->H != 0 || p->K < 1 ||
      p->V < 1)
    return KDA_ERR_SHAPE;
  const long long C = 2LL * p->H * p->K + (long long)p->HV * p->V;
  if (C > 0x7fffffffLL || (long long)p->N * p->T * C > 0x7fffffffLL * 64LL) return KDA_ERR_SHAPE;
  if ((long long)p->N * p->HV * 8 > 0x7fffffffLL) return KDA_ERR_SHAPE;
  if ((long long)p->N * p->T > 0x7fffffffLL / 2) return KDA_ERR_SHAPE;
  if (!supported_kv(p->K, p->V)) return KDA_ERR_UNSUPPORTED;
  if (p->in_dtype != KDA_F32 && p->in_dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
  if (p->gate_mode != KDA_GATE_SOFTPLUS && p->gate_mode != KDA_GATE_SAFE) return KDA_ERR_UNSUPPORTED;
  if (p->variant < KDA_VARIANT_AUTO || p->variant > KDA_VARIANT_LARGE) return KDA_ERR_UNSUPPORTED;
  if (!(p->softplus_beta > 0.0f) || !(p->l2norm_eps >= 0.0f) || p->scale != p->scale) return KDA_ERR_SHAPE;
  if (p->store_policy < 0 || p->store_policy > 2) return KDA_ERR_UNSUPPORTED;
  if (p->max_wg_per_cu != 0 && p->max_wg_per_cu != 1 && p->max_wg_per_cu != 2 && p->max_wg_per_cu != 4 &&
      p->max_wg_per_cu != 6 && p->max_wg_per_cu != 8)
    return KDA_ERR_UNSUPPORTED;
  if (p->column_groups != 0) {
    // groups of 32 or 64 columns splitting a whole-V workgroup (K = V = 128)
    const int wt = p->tile_columns != 0 ? p->tile_columns : p->variant == KDA_VARIANT_SMALL ? 32 : 128;
    const bool ok = p->column_groups == 1 ||
                    (p->K == 128 && p->V == 128 && wt == 128 && (p->column_groups == 2 || p->column_groups == 4) &&
                     !(p->in_dtype == KDA_F32 && p->T > 8));
    if (!ok) return KDA_ERR_UNSUPPORTED;
  }
  if (p->tile_columns != 0) {
    const bool ok = p->K == 128 && p->V == 128 &&
                    (p->tile_columns == 32 || p->tile_columns == 64 || p->tile_columns == 128);
    if (!ok) return KDA_ERR_UNSUPPORTED;
  }
  if (p->schedule < 0 || p->schedule > 3) return KDA_ERR_UNSUPPORTED;
  if (p->unit_order < 0 || p->unit_order > 2) return KDA_ERR_UNSUPPORTED;
  if (p->prefetch < 0 || p->prefetch > 2) return KDA_ERR_UNSUPPORTED;
  if (p->schedule == 3) {
    // the stream: whole-V workgroups of one column group, one per CU, K = V = 128, T <= 8
    const int wt = p->tile_columns != 0 ? p->tile_columns : p->variant == KDA_VARIANT_SMALL ? 32 : 128;
    if (p->K != 128 || p->V != 128 || wt != 128 || p->T > 8 || p->column_groups > 1 || p->max_wg_per_cu > 1)
      return KDA_ERR_UNSUPPORTED;
  }
  if (p->schedule == 2) {
    // the queue runs whole-V workgroups
    bool ok = true;
    if (p->K == 128) {
      const int wt = p->tile_columns != 0 ? p->tile_columns : p->variant == KDA_VARIANT_SMALL ? 32 : 128;
      ok = wt == 128 && !(p->in_dtype == KDA_F32 && p->T > 8);
    } else if (p->K == 64) {
      ok = p->variant != KDA_VARIANT_SMALL;
    }
    if (!ok) return KDA_ERR_UNSUPPORTED;
  }
  return KDA_OK;
}

size_t kda_workspace_bytes(const kda_verify_params* p) {
  if (check_params(p) != KDA_OK) return 0;
  // an arrival counter per (sequence, q/k head), then the queue's ticket and leave counts
  const size_t words = (size_t)p->N * p->H + 2;
  return (words * 4 + 255) / 256 * 256;
}

int32_t kda_select_variant(const kda_verify_params* p) {
  kda_status st = check_params(p);
  if (st != KDA_OK) return st;
  if (p->tile_columns != 0) return p->tile_columns == p->V ? KDA_VARIANT_LARGE : KDA_VARIANT_SMALL;
  if (p->variant != KDA_VARIANT_AUTO) return p->variant;
  return choose_tile(p).vt < p->V ? KDA_VARIANT_SMALL : KDA_VARIANT_LARGE;
}

kda_status kda_select_launch(const kda_verify_params* p, int32_t* tile_columns, int32_t* store_policy,
                             int32_t* max_wg_per_cu, int32_t* column_groups, int32_t* schedule,
                             int32_t* unit_order, int32_t* prefetch) {
  const kda_status st = check_params(p);
  if (st != KDA_OK) return st;
  const Tile t = choose_tile(p);
  if (tile_columns) *tile_columns = t.vt;
  if (store_policy) *store_policy = t.stp == kStoreNTDev ? 2 : 1;
  if (max_wg_per_cu) *max_wg_per_cu = t.occ;
  if (column_groups) *column_groups = t.g;
  if (schedule) *schedule = t.stream ? 3 : t.queue ? 2 : 1;
  if (unit_order) *unit_order = t.order;
  if (prefetch) *prefetch = t.stream ? t.prefetch : 0;
  return KDA_OK;
}

}  // extern "C"

namespace kda {

// Pool rows and index arrays of a call; the identity when pools == NULL.
struct PoolView {
  const int32_t* cs_idx = nullptr;
  const int32_t* st_idx = nullptr;
  const int32_t* in_idx = nullptr;
  size_t cs_slots, st_slots, in_slots;
};

kda_status pool_view(const kda_verify_params* p, const kda_pool_desc* pools, PoolView* v) {
  v->cs_slots = v->st_slots = v->in_slots = (size_t)p->N;
  if (!pools) return KDA_OK;
  if (pools->conv_state_slots < 1 || pools->state_slots < 1 || pools->intermediate_slots < 1) return KDA_ERR_SHAPE;
  if ((long long)pools->state_slots * p->HV * 8 > 0x7fffffffLL) return KDA_ERR_SHAPE;
  const int32_t* idx[] = {pools->conv_state_indices, pools->cache_indices, pools->intermediate_state_indices};
  for (const int32_t* q : idx)
    if (reinterpret_cast<uintptr_t>(q) & 3u) return KDA_ERR_ALIGN;
  v->cs_idx = pools->conv_state_indices;
  v->st_idx = pools->cache_indices;
  v->in_idx = pools->intermediate_state_indices;
  // a NULL index array is the identity, which needs at least N rows
  v->cs_slots = pools->conv_state_slots;
  v->st_slots = pools->state_slots;
  v->in_slots = pools->intermediate_slots;
  if ((!v->cs_idx && v->cs_slots < (size_t)p->N) || (!v->st_idx && v->st_slots < (size_t)p->N) ||
      (!v->in_idx && v->in_slots < (size_t)p->N))
    return KDA_ERR_SHAPE;
  return KDA_OK;
}

Range rg(const void* q, size_t bytes) {
  uintptr_t lo = reinterpret_cast<uintptr_t>(q);
  return Range{lo, lo + bytes};
}

// Written ranges must not overlap each other or any read range.
bool any_alias(const Range* in, size_t nin, const Range* out, size_t nout) {
  for (size_t i = 0; i < nout; ++i) {
    for (size_t j = i + 1; j < nout; ++j)
      if (overlap(out[i], out[j])) return true;
    for (size_t j = 0; j < nin; ++j)
      if (overlap(out[i], in[j])) return true;
  }
  return false;
}

kda_status launch_verify(const kda_verify_params* p, const PoolView& pv, const void* mixed_qkv,
                         const void* conv_weight, void* conv_state, const void* gate, const float* A_log,
                         const float* dt_bias, const void* beta, const float* state, void* o, float* inter_ssm,
                         void* conv_window, void* workspace, hipStream_t stream, bool pre);

kda_status validate_verify(const kda_verify_params* p, const kda_pool_desc* pools, PoolView* pv,
                           const void* mixed_qkv, const void* conv_weight, const void* conv_state, const void* gate,
                           const float* A_log, const float* dt_bias, const void* beta, const float* state,
                           const void* o, const float* inter_ssm, const void* conv_window, const void* workspace,
                           size_t workspace_bytes) {
  kda_status st = check_params(p);
  if (st != KDA_OK) return st;
  if ((st = pool_view(p, pools, pv)) != KDA_OK) return st;
  if (p->N == 0) return KDA_OK;
  const void* ptrs[] = {mixed_qkv, conv_weight, conv_state, gate, A_log, dt_bias,
                        beta,      state,       o,          inter_ssm, conv_window, workspace};
  for (const void* q : ptrs)
    if (!q) return KDA_ERR_NULL;
  for (const void* q : ptrs)
    if (misaligned(q)) return KDA_ERR_ALIGN;
  if (workspace_bytes < kda_workspace_bytes(p)) return KDA_ERR_WORKSPACE;

  const size_t s = p->in_dtype == KDA_BF16 ? 2 : 4;
  const size_t N = p->N, T = p->T, HV = p->HV, K = p->K, V = p->V;
  const size_t C = 2 * (size_t)p->H * K + HV * V;
  const Range in[] = {rg(mixed_qkv, s * N * T * C),
                      rg(conv_weight, s * C * 4),
                      rg(gate, s * N * T * HV * K),
                      rg(A_log, 4 * HV),
                      rg(dt_bias, 4 * HV * K),
                      rg(beta, s * N * T * HV),
                      rg(state, 4 * pv->st_slots * HV * K * V),
                      rg(pv->cs_idx, pv->cs_idx ? 4 * N : 0),
                      rg(pv->st_idx, pv->st_idx ? 4 * N : 0),
                      rg(pv->in_idx, pv->in_idx ? 4 * N : 0)};
  const Range out[] = {rg(conv_state, s * pv->cs_slots * C * 3), rg(o, s * N * T * HV * V),
                       rg(inter_ssm, 4 * pv->in_slots * T * HV * K * V), rg(conv_window, s * pv->in_slots * T * C * 3),
                       rg(workspace, kda_workspace_bytes(p))};
  if (any_alias(in, sizeof(in) / sizeof(in[0]), out, sizeof(out) / sizeof(out[0]))) return KDA_ERR_ALIAS;
  return KDA_OK;
}

}  // namespace kda

extern "C" {

kda_status kda_validate(const kda_verify_params* p, const void* mixed_qkv, const void* conv_weight,
                        const void* conv_state, const void* gate, const float* A_log, const float* dt_bias,
                        const void* beta, const float* state, const void* o, const float* inter_ssm,
                        const void* conv_window, const void* workspace, size_t workspace_bytes) {
  PoolView pv;
  return validate_verify(p, nullptr, &pv, mixed_qkv, conv_weight, conv_state, gate, A_log, dt_bias, beta, state, o,
                         inter_ssm, conv_window, workspace, workspace_bytes);
}

kda_status kda_conv_verify_decode_pooled(const kda_verify_params* p, const kda_pool_desc* pools,
                                         const void* mixed_qkv, const void* conv_weight, void* conv_state,
                                         const void* gate, const float* A_log, const float* dt_bias,
                                         const void* beta, const float* state, void* o, float* inter_ssm,
                                         void* conv_window, void* workspace, size_t workspace_bytes,
                                         hipStream_t stream) {
  PoolView pv;
  kda_status st = validate_verify(p, pools, &pv, mixed_qkv, conv_weight, conv_state, gate, A_log, dt_bias, beta,
                                  state, o, inter_ssm, conv_window, workspace, workspace_bytes);
  if (st != KDA_OK) return st;
  if (p->N == 0) return KDA_OK;
  return launch_verify(p, pv, mixed_qkv, conv_weight, conv_state, gate, A_log, dt_bias, beta, state, o, inter_ssm,
                       conv_window, workspace, stream, false);
}

}  // extern "C"

namespace kda {

kda_status launch_verify(const kda_verify_params* p, const PoolView& pv, const void* mixed_qkv,
                         const void* conv_weight, void* conv_state, const void* gate, const float* A_log,
                         const float* dt_bias, const void* beta, const float* state, void* o, float* inter_ssm,
                         void* conv_window, void* workspace, hipStream_t stream, bool pre) {
  Tile tl = choose_tile(p);
  if (pre) tl.queue = tl.stream = false;  // the unfused form keeps one workgroup per unit
  LaunchFn fn = pick_launch(p, tl, pre);
  if (!fn) return KDA_ERR_UNSUPPORTED;
  Args a;
  a.mixed_qkv = mixed_qkv;
  a.conv_weight = conv_weight;
  a.conv_state = conv_state;
  a.gate = gate;
  a.A_log = A_log;
  a.dt_bias = dt_bias;
  a.beta = beta;
  a.state = state;
  a.o = o;
  a.inter_ssm = inter_ssm;
  a.conv_window = conv_window;
  a.counters = static_cast<uint32_t*>(workspace);
  a.cs_idx = pv.cs_idx;
  a.st_idx = pv.st_idx;
  a.in_idx = pv.in_idx;
  a.cs_slots = (int)pv.cs_slots;
  a.st_slots = (int)pv.st_slots;
  a.in_slots = (int)pv.in_slots;
  a.N = p->N;
  a.T = p->T;
  a.H = p->H;
  a.HV = p->HV;
  a.C = 2 * p->H * p->K + p->HV * p->V;
  a.g = p->HV / p->H;
  a.group = 0;
  a.order = kOrderXcdRanges;
  a.gate_mode = p->gate_mode;
  a.lower_bound = p->lower_bound;
  a.softplus_beta = p->softplus_beta;
  a.softplus_threshold = p->softplus_threshold;
  a.scale = p->scale > 0.0f ? p->scale : 1.0f / sqrtf((float)p->K);
  a.eps = p->l2norm_eps;
  return fn(a, tl, stream) == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

}  // namespace kda

extern "C" {

kda_status kda_conv_verify_decode_unfused(const kda_verify_params* p, const kda_pool_desc* pools,
                                          const void* mixed_qkv, const void* conv_weight, void* conv_state,
                                          const void* gate, const float* A_log, const float* dt_bias,
                                          const void* beta, const float* state, void* o, float* inter_ssm,
                                          void* conv_window, void* act, void* workspace, size_t workspace_bytes,
                                          hipStream_t stream) {
  PoolView pv;
  kda_status st = validate_verify(p, pools, &pv, mixed_qkv, conv_weight, conv_state, gate, A_log, dt_bias, beta,
                                  state, o, inter_ssm, conv_window, workspace, workspace_bytes);
  if (st != KDA_OK) return st;
  if (p->schedule >= 2) return KDA_ERR_UNSUPPORTED;
  if (p->N == 0) return KDA_OK;
  if (!act) return KDA_ERR_NULL;
  if (misaligned(act)) return KDA_ERR_ALIGN;
  const size_t s = p->in_dtype == KDA_BF16 ? 2 : 4;
  const size_t C = 2 * (size_t)p->H * p->K + (size_t)p->HV * p->V;
  const Range act_r = rg(act, 4 * (size_t)p->N * p->T * C);
  const void* others[] = {mixed_qkv, conv_weight, conv_state, gate, A_log, dt_bias, beta, state, o, inter_ssm,
                          conv_window, workspace};
  const size_t sizes[] = {s * p->N * p->T * C, s * C * 4, s * pv.cs_slots * C * 3, s * p->N * p->T * p->HV * p->K,
                          4 * (size_t)p->HV, 4 * (size_t)p->HV * p->K, s * p->N * p->T * p->HV,
                          4 * pv.st_slots * p->HV * p->K * p->V, s * p->N * p->T * p->HV * p->V,
                          4 * pv.in_slots * p->T * p->HV * p->K * p->V, s * pv.in_slots * p->T * C * 3,
                          kda_workspace_bytes(p)};
  for (size_t i = 0; i < sizeof(others) / sizeof(others[0]); ++i)
    if (overlap(act_r, rg(others[i], sizes[i]))) return KDA_ERR_ALIAS;
  ConvArgs c;
  c.x = mixed_qkv;
  c.w = conv_weight;
  c.conv_state = conv_state;
  c.conv_window = conv_window;
  c.act = act;
  c.cs_idx = pv.cs_idx;
  c.st_idx = pv.st_idx;
  c.in_idx = pv.in_idx;
  c.cs_slots = (int)pv.cs_slots;
  c.st_slots = (int)pv.st_slots;
  c.in_slots = (int)pv.in_slots;
  c.N = p->N;
  c.T = p->T;
  c.C = (int)C;
  void* cargs[] = {&c};
  const void* ck = p->in_dtype == KDA_BF16 ? reinterpret_cast<const void*>(&kda_conv_silu_kernel<uint16_t>)
                                           : reinterpret_cast<const void*>(&kda_conv_silu_kernel<uint32_t>);
  if (hipLaunchKernel(ck, dim3((unsigned)((C + 255) / 256), (unsigned)p->N), dim3(256), cargs, 0, stream) !=
      hipSuccess)
    return KDA_ERR_LAUNCH;
  return launch_verify(p, pv, act, conv_weight, conv_state, gate, A_log, dt_bias, beta, state, o, inter_ssm,
                       conv_window, workspace, stream, true);
}

kda_status kda_conv_verify_decode(const kda_verify_params* p, const void* mixed_qkv, const void* conv_weight,
                                  void* conv_state, const void* gate, const float* A_log, const float* dt_bias,
                                  const void* beta, const float* state, void* o, float* inter_ssm,
                                  void* conv_window, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return kda_conv_verify_decode_pooled(p, nullptr, mixed_qkv, conv_weight, conv_state, gate, A_log, dt_bias, beta,
                                       state, o, inter_ssm, conv_window, workspace, workspace_bytes, stream);
}

kda_status kda_verify_commit(const kda_verify_params* p, const kda_pool_desc* pools, const int32_t* accepted,
                             const float* inter_ssm, const void* conv_window, float* state, void* conv_state,
                             hipStream_t stream) {
  kda_status st = check_params(p);
  if (st != KDA_OK) return st;
  PoolView pv;
  if ((st = pool_view(p, pools, &pv)) != KDA_OK) return st;
  if (p->N == 0) return KDA_OK;
  const void* ptrs[] = {accepted, inter_ssm, conv_window, state, conv_state};
  for (const void* q : ptrs)
    if (!q) return KDA_ERR_NULL;
  for (const void* q : ptrs)
    if (misaligned(q)) return KDA_ERR_ALIGN;
  const size_t s = p->in_dtype == KDA_BF16 ? 2 : 4;
  const size_t N = p->N, T = p->T, HV = p->HV, K = p->K, V = p->V;
  const size_t C = 2 * (size_t)p->H * K + HV * V;
  const Range in[] = {rg(accepted, 4 * N),
                      rg(inter_ssm, 4 * pv.in_slots * T * HV * K * V),
                      rg(conv_window, s * pv.in_slots * T * C * 3),
                      rg(pv.cs_idx, pv.cs_idx ? 4 * N : 0),
                      rg(pv.st_idx, pv.st_idx ? 4 * N : 0),
                      rg(pv.in_idx, pv.in_idx ? 4 * N : 0)};
  const Range out[] = {rg(state, 4 * pv.st_slots * HV * K * V), rg(conv_state, s * pv.cs_slots * C * 3)};
  if (any_alias(in, sizeof(in) / sizeof(in[0]), out, sizeof(out) / sizeof(out[0]))) return KDA_ERR_ALIAS;
  CommitArgs a;
  a.accepted = accepted;
  a.inter_ssm = inter_ssm;
  a.conv_window = conv_window;
  a.state = state;
  a.conv_state = conv_state;
  a.cs_idx = pv.cs_idx;
  a.st_idx = pv.st_idx;
  a.in_idx = pv.in_idx;
  a.cs_slots = (int)pv.cs_slots;
  a.st_slots = (int)pv.st_slots;
  a.in_slots = (int)pv.in_slots;
  a.N = p->N;
  a.T = p->T;
  a.HV = p->HV;
  a.C = (int)C;
  a.kv4 = (int)(K * V / 4);
  a.cs_vec = (int)(C * 3 * s / 16);
  // Up to 1024 units, 256 threads with 16 vectors each; beyond, 1024 threads with 4 each.
  // Measured on MI355X against one 256-thread shape with 8 vectors per round, the whole
  // conv row copied by the hv == 0 WG and device-scope streaming stores (cache evicted
  // between calls): 29.7 -> 15.9 us at 512 units (small_batch), 66.7 -> 55.8 us at 2048
  // (gva), 220 -> 191 us at 8192 (large_batch), 792 -> 725 us at 32768 (max_bandwidth); at
  // 256-1024 units the small shape was 14-23 % ahead of the large one, from 2048 units the
  // large one 6-9 % ahead of the small; device-scope stores lost 4-25 % on the small shape
  // and were within 1.5 % either way on the large one.
  const bool small = N * HV <= 1024;
  const void* fn = small ? reinterpret_cast<const void*>(&kda_commit_kernel<256, 16>)
                         : reinterpret_cast<const void*>(&kda_commit_kernel<1024, 4>);
  void* args[] = {&a};
  return hipLaunchKernel(fn, dim3((unsigned)(N * HV)), dim3(small ? 256 : 1024), args, 0, stream) == hipSuccess
             ? KDA_OK
             : KDA_ERR_LAUNCH;
}

kda_status kda_workspace_reset(void* workspace, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return KDA_OK;
  if (!workspace) return KDA_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(workspace) & 3u) || (bytes & 3u)) return KDA_ERR_ALIGN;
  return launch_zero_words(static_cast<uint32_t*>(workspace), bytes / 4, stream) == hipSuccess ? KDA_OK
                                                                                              : KDA_ERR_LAUNCH;
}

kda_status kda_conv_verify_decode_noalloc(const kda_verify_params* p, const void* mixed_qkv, const void* conv_weight,
                                          void* conv_state, const void* gate, const float* A_log,
                                          const float* dt_bias, const void* beta, const float* state, void* o,
                                          float* inter_ssm, void* conv_window, hipStream_t stream) {
  kda_status st = check_params(p);
  if (st != KDA_OK) return st;
  const size_t need = kda_workspace_bytes(p);
  if (need > KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_SCRATCH;
  if (p->N == 0) return KDA_OK;
  uint32_t* ws = nullptr;
  if (scratch_on_current_device(&ws) != hipSuccess) return KDA_ERR_LAUNCH;
  PoolView pv;
  st = validate_verify(p, nullptr, &pv, mixed_qkv, conv_weight, conv_state, gate, A_log, dt_bias, beta, state, o,
                       inter_ssm, conv_window, ws, KDA_NOALLOC_SCRATCH_BYTES);
  if (st != KDA_OK) return st;
  // the counters must start at zero; the previous call on this GPU normally left them so,
  // but one that did not run to completion may not have
  if (launch_zero_words(ws, need / 4, stream) != hipSuccess) return KDA_ERR_LAUNCH;
  return launch_verify(p, pv, mixed_qkv, conv_weight, conv_state, gate, A_log, dt_bias, beta, state, o, inter_ssm,
                       conv_window, ws, stream, false);
}

const char* kda_status_string(int32_t status) {
  switch (status) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULL: return "a required pointer is NULL";
    case KDA_ERR_SHAPE: return "a size is out of range or inconsistent";
    case KDA_ERR_UNSUPPORTED: return "unsupported (K, V), dtype, gate mode or variant";
    case KDA_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
    case KDA_ERR_WORKSPACE: return "workspace missing or too small";
    case KDA_ERR_LAUNCH: return "kernel launch failed";
    case KDA_ERR_ALIAS: return "an output buffer overlaps another buffer";
    case KDA_ERR_SCRATCH: return "the shape needs more counters than the allocation-free call's static scratch holds";
    default: return "unknown status";
  }
}

}  // extern "C"
