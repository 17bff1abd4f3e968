// Internal declarations shared by the host API and the kernel translation units.
// Nothing here is part of the public ABI (include/lcs.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lcs {

// ---------------------------------------------------------------------------
// Attention (verify, sparse token lists, sparse block lists)
// ---------------------------------------------------------------------------
enum AttnMode : int32_t {
  MODE_DENSE = 0,          // verify: every cache position [0, L + n_q)
  MODE_LIST_SHARED = 1,    // sparse: one token list per sequence
  MODE_LIST_PER_HEAD = 2,  // sparse: one token list per (sequence, KV head)
  MODE_BLOCK = 3,          // sparse: per-row block lists, merged into a union
  MODE_NSA = 4             // NSA: compression, selection (union plan) and window branches
};

// NSA branches, in the order of their split ranges in a launch and of the gates
enum NsaBranch : int32_t { BR_CMP = 0, BR_SLC = 1, BR_WIN = 2 };

constexpr int kStepTokens = 32;   // tokens consumed per inner step of a wave
constexpr int kWaves = 4;         // waves per workgroup (one token stream each)
constexpr int kMaxRowsPerWG = 48; // q-rows (n_q * G) handled by one workgroup: three 16-row
                                  // tiles, the most whose accumulators fit one wave's registers
constexpr int kMaxSplits = 128;   // split-K partials per (sequence, KV head, row chunk)
constexpr int kDefaultCUs = 256;  // MI355X compute units; used when the device cannot be queried

struct AttnArgs {
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* bt;
  int32_t num_pages, lg_page, max_pages, Hkv;
  const uint16_t* q;
  int32_t B, n_q, Hq, G, rows, n_rc;
  int32_t mode;
  // dense verify
  const int32_t* prefix_len;
  int32_t max_prefix_len;
  // dense: tree mask; sparse: tail mask.  [B][n_q] or null
  const uint64_t* rowmask;
  // sparse lists
  const int32_t* indices;
  const int32_t* counts;
  int32_t cap;
  const int32_t* tail_begin;
  const int32_t* tail_len;
  int32_t max_tail_len;   // tail_len values above it are clamped
  int32_t phys;           // token lists hold physical slots (page * page_size + slot), not positions
  // block-union plan (workspace)
  const int32_t* ublk;
  const uint64_t* umask;
  const int32_t* ucount;
  int32_t ucap;
  float scale, scale_log2;
  // Collected logit rows (dense only).  Verifier row i is collected iff bit i of cmask
  // is set; it goes to slot popcount(cmask below i) of the n_cl slots per head, to the
  // other slot of two when cswap is set, and to slots 0 and 1 when cdup is set.
  uint64_t cmask;
  int32_t n_cl, cswap, cdup;
  float* logits;
  int64_t logits_ld;
  int32_t lvec4;   // logits rows 16-byte aligned (16-byte stores allowed)
  // Per-KV-head partial scores instead of logits (dense only): [B][Hkv][scores_ld],
  // the sum over the group's heads, ascending, of (row0 + row1) logits
  float* scores;
  int64_t scores_ld;
  // NSA: compressed cache [B][Hkv][max_cmp][d], compression block length and stride,
  // window length, gates [B][n_q][Hq][3]; the launch's splits are ns0 compression splits,
  // then ns1 selection splits, then ns2 window splits.  approx: the union plan gives
  // every row of a group the whole union (approximate grouping).
  const uint16_t* ck;
  const uint16_t* cv;
  int32_t max_cmp, cmp_len, cmp_stride, window;
  const float* gates;
  int32_t ns0, ns1, ns2;
  int32_t approx;
  // split-K
  float* part;
  int32_t n_split;
  int32_t T_max;   // step bound of the launch (list modes split it across waves)
  // final outputs
  float* out;
  float* lse;
};

struct AttnPlan {
  int32_t D, QT, rows, n_rc, n_split, T_max;
  int32_t ns_br[3];   // MODE_NSA: splits of each branch (sum = n_split)
  size_t part_bytes, ublk_bytes, umask_bytes, ucount_bytes, total_bytes;
};

// Byte layout of a block-union plan for (B, Hkv) pairs of n_q rows x cap blocks:
// ublk int32 [B*Hkv][n_q*cap], umask uint64 [B*Hkv][n_q*cap], ucount int32 [B*Hkv].
struct UnionLayout {
  size_t ublk_bytes, umask_bytes, ucount_bytes, total_bytes;
};
UnionLayout union_layout(int32_t B, int32_t Hkv, int32_t n_q, int32_t cap);

// NSA split policy and workspace (split-K partials only; the union plan is the caller's).
AttnPlan attn_plan_nsa(int32_t B, int32_t n_q, int32_t Hq, int32_t Hkv, int32_t d, int32_t page_size,
                       int32_t cap, int32_t max_tail_len, int32_t max_cmp, int32_t window, int32_t cus);

// Build the block-union plan of a.indices / a.counts into a.ublk / a.umask / a.ucount.
hipError_t union_launch(const AttnArgs& a, hipStream_t stream);

// Compressed cache: row i of (b, g) = bf16 mean of positions [i*stride, i*stride + len).
hipError_t compress_launch(const AttnArgs& a, int32_t d, int32_t B, const int32_t* prefix_len, uint16_t* kc,
                           uint16_t* vc, hipStream_t stream);

// Split policy and workspace layout; identical on every call with the same sizes on the
// same device.  cus = compute units of the current device (device_cus()).
AttnPlan attn_plan(int32_t mode, int32_t B, int32_t n_q, int32_t Hq, int32_t Hkv, int32_t d,
                   int32_t page_size, int32_t max_prefix_len, int32_t cap, int32_t max_tail_len,
                   int32_t cus);

// Compute units of the current HIP device, read once per device (kDefaultCUs when no
// device can be queried, e.g. for a workspace query on a machine without a GPU).
int32_t device_cus();

// Launch the attention kernels on `stream`.  Returns hipSuccess or the launch error.
hipError_t attn_launch(const AttnPlan& plan, AttnArgs args, void* workspace, hipStream_t stream);

// ---------------------------------------------------------------------------
// Selection
// ---------------------------------------------------------------------------
enum SelMode : int32_t { LCS_SEL_SHARED = 0, LCS_SEL_PER_HEAD = 1, LCS_SEL_BLOCK = 2 };

constexpr int kScorePos = 512;         // positions per workgroup of the score pass
constexpr int kItemChunk = 4096;       // items per workgroup of the collect and emit passes
constexpr int kMaxItemChunks = 4096;   // items < 2^24
constexpr int kHistBins = 4096;        // first radix digit: top 12 bits of the key

// Position score of a set (the selection passes are identical for both):
//   SCORE_LOGIT_SUM:   per head, the collected rows' logits summed in slot order;
//   SCORE_SOFTMAX_WT:  per head, the rows' softmax weights exp(logit - lse) summed.
enum ScoreKind : int32_t { SCORE_LOGIT_SUM = 0, SCORE_SOFTMAX_WT = 1 };

struct SelArgs {
  const float* logits;
  int64_t ld;
  int32_t n_rows, kind;    // logit rows per head; ScoreKind
  const float* lse;        // SCORE_SOFTMAX_WT: [B][n_q][Hq]
  int32_t n_q;
  uint64_t rows_mask;      // SCORE_SOFTMAX_WT: slot c holds verifier row = c-th set bit
  int32_t B, Hq, Hkv, G, n_sets, mode;
  const int32_t* prefix_len;
  int32_t max_len;
  int32_t top_k, n_sink, n_recent, lg_bs, vec4;
  int32_t block_lse;       // block mode: score a block by log-sum-exp instead of max
  const int32_t* bt;       // non-null: emit physical slots bt[b][p / P] * P + p % P, not positions
  int32_t max_pages, lg_page;
  int32_t* indices;
  int32_t* counts;
  int32_t cap;
  // workspace
  uint32_t* keys;        // [NS][item_cap]
  uint32_t* hist;        // [NS][kHistBins]
  uint32_t* cand_count;  // [NS]
  uint64_t* cand;        // [NS][item_cap]
  uint32_t* chunk_above; // [NS][n_chunks]
  uint64_t* thr;         // [NS][2]
  uint64_t* marker;      // histograms left clean by the last call of this layout
  uint64_t marker_value; // the value that says so for this call's layout
  int32_t item_cap, n_chunks, n_pos_chunks;
  int32_t score_iters;   // 512-position chunks one score workgroup covers (1 in block mode)
};

struct SelPlan {
  int32_t n_sets, item_cap, n_chunks, n_pos_chunks, score_iters;
  int32_t fin_threads;   // threads of a finish workgroup (256, 512 or 1024)
  size_t keys_bytes, hist_bytes, cc_bytes, cand_bytes, ca_bytes, thr_bytes, mk_bytes, total_bytes;
};

// cus: compute units of the device (0: the MI355X's 256); reads: score values read per
// position (heads of a set x rows; 0: many).  Only the launch shape depends on either.
SelPlan select_plan(int32_t B, int32_t Hq, int32_t Hkv, int32_t mode, int32_t max_len,
                    int32_t block_size, int32_t cus = 0, int32_t reads = 0);

hipError_t select_launch(const SelPlan& plan, SelArgs args, void* workspace, hipStream_t stream);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---------------------------------------------------------------------------
// Wave primitives (64 lanes, every lane active).  None goes through LDS: a shuffle
// through LDS waits for the LDS return at each of its steps.
// ---------------------------------------------------------------------------
// Inclusive prefix sum.  Within each 16-lane row, four DPP row shifts (a lane whose
// source lies before its row's start adds 0); then each row adds the totals of the rows
// below it, read with readlane.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  int x = (int)v;
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(x, 15);
  const int r1 = __builtin_amdgcn_readlane(x, 31);
  const int r2 = __builtin_amdgcn_readlane(x, 47);
  const int row = (threadIdx.x & 63) >> 4;
  x += (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
  return (uint32_t)x;
}

// Butterfly all-reduce over lane xor 32, 16, 8, 4, 2, 1, in that order.  The gfx950
// half and row swaps (v_permlane32_swap, v_permlane16_swap) return both members of the
// lane xor 32 (xor 16) pair, so op(first, second) combines a lane with its partner.
// Lane xor 8 is row_ror:8 (rotating a 16-lane row by 8); lane xor 4 is row_ror:4 once
// lanes r and r ^ 8 hold the same value, which the xor-8 step leaves; xor 2 and xor 1
// are quad permutations.  Each step combines the same pair of values as the
// xor-shuffle butterfly, so with an op that gives one result for either operand order
// (a sum; a max, up to the sign of a zero) every lane ends with the same value, bit for
// bit the shuffle butterfly's.
template <typename Op>
__device__ __forceinline__ float wave_bfly_f32(float v, Op op) {
  const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = op(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
  const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = op(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
  v = op(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false)));
  v = op(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xf, 0xf, false)));
  v = op(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xf, 0xf, false)));
  v = op(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xf, 0xf, false)));
  return v;
}
__device__ __forceinline__ float wave_sum_f32(float v) {
  return wave_bfly_f32(v, [](float a, float b) { return a + b; });
}
__device__ __forceinline__ float wave_max_f32(float v) {
  return wave_bfly_f32(v, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ uint32_t wave_or_u32(uint32_t v) {
  const auto s32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  v = s32[0] | s32[1];
  const auto s16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = s16[0] | s16[1];
  v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xf, 0xf, false);
  v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xf, 0xf, false);
  v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xf, 0xf, false);
  v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xf, 0xf, false);
  return v;
}
// lane + lane ^ 16, then + lane ^ 32 (the xor-shuffle pair sums in that order)
__device__ __forceinline__ float sum_x16_x32(float v) {
  const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
  const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
}

}  // namespace lcs
