// Paged GQA attention kernels for gfx950: dense verify with Collect-2-Query logits,
// sparse draft attention over token lists, and block-sparse grouped rows with
// overlap-aware union loads.
//
// What is computed
//  * Vegas page, "The pith" / "Core claim": verification is full attention of the
//    k+1 verifier rows over the whole KV cache; the pre-softmax logits of the first
//    draft row and the bonus row are written out (Figure 6 caption: two rows only,
//    so the side traffic stays constant in k).  The same kernel also collects any
//    other set of rows, or sums the two rows over each KV group's heads and writes
//    one score row per KV head instead.
//  * Vegas page, "The pith": drafting attends to the selected prefix entries only.
//  * SSV page, section 4.2 (exact merged-schedule variant) and Figure 5: grouped
//    verifier rows with different block sets load each shared block once; each row
//    keeps its own selection and its own causal boundary (Figure 6 text).
//
// How (gfx950, wave64, MFMA, LDS DMA)
//  * One workgroup = 4 waves = one (sequence, KV head, row chunk, split).  Every
//    q-row of the KV group (n_q verifier rows x G query heads) is a row of the MFMA
//    tile, so each K/V byte fetched from HBM serves all G heads and all n_q rows.
//  * A wave owns a contiguous run of 32-token steps.  Every byte it streams goes
//    global -> LDS with global_load_lds_dwordx4 (K/V tiles) or _dword (index-list
//    and block-table entries) into per-wave LDS slots, two steps ahead, with the
//    vmcnt waits placed by hand.  No vector register waits on global memory inside
//    the loop, so the wave keeps 32 KB in flight while it computes.
//  * Each lane DMAs exactly the 16-byte pieces it later needs as MFMA operands:
//    S^T = K Q^T on v_mfma_f32_16x16x32_bf16 takes K rows (lane = token, 8
//    contiguous dims) as A; O^T = V^T P^T takes 8 tokens x 8 dims per lane,
//    transposed in registers (v_perm), as A, and P straight from the S^T
//    accumulator layout as B.  P is split into bf16 hi + lo parts so the PV product
//    keeps ~16 mantissa bits of the softmax weights.  d = 64 uses the same operand
//    layout with the upper half of the V^T rows idle.
//  * Token metadata (row index, row-visibility mask) for a window of kMW steps is
//    built one window ahead in three stages spread over three steps.
//  * Online softmax in base 2 with the running max and sum per q-row kept in the
//    lane that owns the row; the 4 waves' states are merged through LDS in a fixed
//    order, and a split-K combine merges the workgroups' partials in a fixed order,
//    so results are bitwise reproducible.
//  * The kernel is HBM-bound by design (arithmetic intensity ~ n_q*G flop/byte, far
//    below the MFMA ridge); MFMA is used because the VALU alone could not keep up
//    with the 36-row verify tile at full bandwidth.
#include "lcs_internal.h"

#include <math.h>

#include <type_traits>

namespace lcs {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

typedef void __attribute__((address_space(3)))* lptr_t;

constexpr uint64_t kAll = ~0ull;
constexpr float kLn2 = 0.693147180559945309417f;
constexpr float kTau = 8.f;   // log2 headroom of the lazily updated softmax reference max

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint64_t shfl64(uint64_t v, int src) {
  uint32_t lo = __shfl((uint32_t)v, src);
  uint32_t hi = __shfl((uint32_t)(v >> 32), src);
  return ((uint64_t)hi << 32) | lo;
}

// max over the four lanes {l, l^16, l^32, l^48} (the 4 lane groups holding one MFMA
// column) with gfx950 permlane swaps: VALU only, no LDS round trip.
__device__ __forceinline__ float fmax2(float a, float b) { return a > b ? a : b; }
// three-input max in one VALU op (fmaxf would first quieten every input); the
// operands are never NaN here: masked entries are -inf, all others are finite
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float colmax4(float v) {
  const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float a = max3f(__uint_as_float(s32[0]), __uint_as_float(s32[1]), __uint_as_float(s32[1]));
  const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(a), false, false);
  return max3f(__uint_as_float(s16[0]), __uint_as_float(s16[1]), __uint_as_float(s16[1]));
}

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// two floats -> packed bf16 pair (x in the low half), round to nearest even, one op
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float x, float y) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){x, y}, bf16x2_t));
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) {
  return __builtin_bit_cast(float, h << 16);
}

// Global -> LDS DMA.  Issued through inline asm so that the compiler's wait-count
// pass, which cannot tell which LDS bytes a DMA writes and would otherwise drain every
// outstanding load before each LDS read, stays out of the pipeline: the waits for
// these loads are placed by hand (wait_vm).  M0 carries the wave-uniform LDS base;
// nothing else in these kernels uses M0.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(lptr_t)p);
}
// 16 bytes per lane from src into LDS at dst + 16 * lane (dst wave-uniform).  NT: the
// K/V rows are read once per call, so the load carries the non-temporal hint (measured
// on the 128K x 8 step: verify 950 -> 913 us, a draft step 35.6 -> 32.5 us).  Launches
// whose row chunks re-read the same K/V (more than 48 q-rows per KV group) load without
// it, so that the re-reads hit the caches.
template <bool NT>
__device__ __forceinline__ void dma16(const void* src, void* dst) {
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(src), "s"(lds_addr(dst))
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds_addr(dst))
                 : "memory", "m0");
}
// 4 bytes per lane from src into LDS at dst + 4 * lane (dst wave-uniform).
__device__ __forceinline__ void dma4(const void* src, void* dst) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(lds_addr(dst))
               : "memory", "m0");
}

// 16-byte store with device scope (sc1): the staged logit runs are written through to
// memory instead of as non-temporal stores; measured on the 128K x 8 step, verify
// 913 -> 892 us for select 68.7 -> 70.4 us and a draft step 32.0 -> 32.5 us.
__device__ __forceinline__ void store_dev_scope(float* dst, f32x4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1" ::"v"(dst), "v"(v) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// compile-time loop: f(integral_constant<int, I>) for I in [B, E)
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

struct SeqInfo {
  int L, cnt, tb, tl, U, T;
  int br;      // NSA: branch of this workgroup
  int cbase;   // NSA compression branch: row of (b, g)'s first compressed block
  const int32_t* list;
  const int32_t* ub;
  const uint64_t* um;
};

// Sequence-level bounds for (b, g); every quantity read from device memory is clamped.
// NSA: cnt = compressed blocks (compression branch) or window prefix tokens (window
// branch); the selection branch reads the union plan like block mode.
template <int MODE>
__device__ __forceinline__ SeqInfo seq_info(const AttnArgs& a, int b, int g, int br = 0) {
  SeqInfo si{};
  const int P = 1 << a.lg_page;
  si.br = br;
  if (MODE == MODE_NSA) {
    si.tb = max(a.tail_begin[b], 0);
    si.tl = min(max(a.tail_len[b], 0), a.max_tail_len);
    if (br == BR_CMP) {
      si.cnt = (si.tb < a.cmp_len) ? 0 : min((si.tb - a.cmp_len) / a.cmp_stride + 1, a.max_cmp);
      si.cbase = (b * a.Hkv + g) * a.max_cmp;
      si.T = (si.cnt + kStepTokens - 1) / kStepTokens;
    } else if (br == BR_SLC) {
      const size_t o = (size_t)(b * a.Hkv + g);
      si.U = min(max(a.ucount[o], 0), a.ucap);
      si.ub = a.ublk + o * a.ucap;
      si.um = a.umask + o * a.ucap;
      si.T = si.U * (P / kStepTokens) + (si.tl + kStepTokens - 1) / kStepTokens;
    } else {
      si.cnt = min(a.window, si.tb);
      si.T = (si.cnt + kStepTokens - 1) / kStepTokens + (si.tl + kStepTokens - 1) / kStepTokens;
    }
    return si;
  }
  if (MODE == MODE_DENSE) {
    si.L = min(max(a.prefix_len[b], 0), a.max_prefix_len);
    si.T = (si.L + a.n_q + kStepTokens - 1) / kStepTokens;
  } else {
    si.tb = a.tail_begin[b];
    si.tl = min(max(a.tail_len[b], 0), a.max_tail_len);
    if (MODE == MODE_BLOCK) {
      const size_t o = (size_t)(b * a.Hkv + g);
      si.U = min(max(a.ucount[o], 0), a.ucap);
      si.ub = a.ublk + o * a.ucap;
      si.um = a.umask + o * a.ucap;
      si.T = si.U * (P / kStepTokens) + (si.tl + kStepTokens - 1) / kStepTokens;
    } else {
      const int nsets = (a.mode == MODE_LIST_SHARED) ? 1 : a.Hkv;
      const int set = (a.mode == MODE_LIST_SHARED) ? 0 : g;
      si.cnt = (a.cap > 0) ? min(max(a.counts[b * nsets + set], 0), a.cap) : 0;
      si.list = a.indices + (size_t)(b * nsets + set) * a.cap;
      si.T = (si.cnt + si.tl + kStepTokens - 1) / kStepTokens;
    }
  }
  return si;
}

// ---------------------------------------------------------------------------
// Token metadata.  For each window of kMW steps a wave builds, one window ahead,
// the K/V row index and the row-visibility mask of every token slot in its LDS
// area: stage A DMAs index-list entries (list mode), stage B DMAs block-table
// entries, stage C turns them into rows, masks and per-step "all visible" flags.
// The stage scratch (indices, pages) lives in the next window's mask buffer.
// ---------------------------------------------------------------------------
constexpr int kMW = 4;                      // steps per metadata window
constexpr int kStageRows = 8;               // collected logit rows (slots x heads) a wave stages
constexpr int kStageSteps = 4;              // steps staged before one flush (512-byte row runs)
constexpr int kStageStride = kStageSteps * 32 + 4;   // floats per staged row: 16 bytes of padding
constexpr int kMT = kMW * kStepTokens;      // token slots per window
constexpr int kTokPerLane = kMT / 64;       // slots each lane handles per stage

struct WaveMeta {
  int32_t row[2][kMT];
  uint64_t vis[2][kMT];     // also stage scratch: int32 index[kMT], int32 page[kMT]
  uint32_t full[2][kMW];
};

// Logical position of slot tok of a window starting at step wbase; jt = tail slot or -1;
// v = row-visibility mask of a non-tail token.  idx = the DMA'd index-list entry.
template <int MODE>
__device__ __forceinline__ void slot_pos(const AttnArgs& a, const SeqInfo& si, int wbase, int w1, int tok,
                                         int idx, int& pos, int& jt, uint64_t& v) {
  const int P = 1 << a.lg_page;
  const int step = wbase + tok / kStepTokens;
  const int t = tok & (kStepTokens - 1);
  pos = -1;
  jt = -1;
  v = 0;
  // block mode: the union entry of each half-wave's step (lanes 0-31 and 32-63 hold
  // different steps), read with wave-uniform loads while every lane is active
  int blk = -1;
  uint64_t bmask = 0;
  if ((MODE == MODE_BLOCK || (MODE == MODE_NSA && si.br == BR_SLC)) && si.U > 0) {
    const int spb = P / kStepTokens;
    const int e_lo = min(__builtin_amdgcn_readfirstlane(step) / spb, si.U - 1);
    const int e_hi = min(__builtin_amdgcn_readlane(step, 32) / spb, si.U - 1);
    const int b_lo = si.ub[max(e_lo, 0)], b_hi = si.ub[max(e_hi, 0)];
    const uint64_t m_lo = si.um[max(e_lo, 0)], m_hi = si.um[max(e_hi, 0)];
    const bool lo_half = (threadIdx.x & 63) < 32;
    blk = lo_half ? b_lo : b_hi;
    bmask = lo_half ? m_lo : m_hi;
  }
  if (step >= w1) return;
  if (MODE == MODE_DENSE) {
    const int u = step * kStepTokens + t;
    if (u < si.L) {
      pos = u;
      v = kAll;
    } else if (u < si.L + a.n_q) {
      pos = u;
      jt = u - si.L;
    }
  } else if (MODE == MODE_NSA && si.br == BR_CMP) {
    const int u = step * kStepTokens + t;      // compressed block index
    if (u < si.cnt) {
      pos = u;
      v = kAll;
    }
  } else if (MODE == MODE_NSA && si.br == BR_WIN) {
    const int pre = (si.cnt + kStepTokens - 1) / kStepTokens;
    if (step < pre) {
      const int u = step * kStepTokens + t;
      if (u < si.cnt) {
        pos = si.tb - si.cnt + u;
        v = kAll;
      }
    } else {
      const int u = (step - pre) * kStepTokens + t;
      if (u < si.tl) {
        pos = si.tb + u;
        jt = u;
      }
    }
  } else if (MODE == MODE_BLOCK || MODE == MODE_NSA) {
    const int spb = P / kStepTokens;
    const int blk_steps = si.U * spb;
    if (step < blk_steps) {
      const int e = step / spb;
      const int p = blk * P + (step - e * spb) * kStepTokens + t;
      if (blk >= 0 && blk < a.max_pages && p < si.tb) {
        pos = p;
        v = bmask;
      }
    } else {
      const int u = (step - blk_steps) * kStepTokens + t;
      if (u < si.tl) {
        pos = si.tb + u;
        jt = u;
      }
    }
  } else {
    const int u = step * kStepTokens + t;
    if (u < si.cnt) {
      pos = idx;
      v = kAll;
    } else if (u - si.cnt < si.tl) {
      jt = u - si.cnt;
      pos = si.tb + jt;
    }
  }
}

// Stage A (list mode): DMA the index-list entry of every slot into scratch index[].
template <int MODE>
__device__ __forceinline__ void meta_stage_a(const AttnArgs& a, const SeqInfo& si, int wbase, int lane,
                                             WaveMeta& wm, int nb) {
  if (MODE != MODE_LIST_SHARED) return;
  int32_t* sidx = reinterpret_cast<int32_t*>(wm.vis[nb]);
#pragma unroll
  for (int r = 0; r < kTokPerLane; ++r) {
    const int tok = lane + 64 * r;
    const int u = (wbase + tok / kStepTokens) * kStepTokens + (tok & (kStepTokens - 1));
    // every lane issues, clamped into the list's cap entries (the block table stands in
    // when cap is 0); the count itself is not needed yet, so this can go out first
    const int32_t* src = (a.cap > 0) ? si.list + min(max(u, 0), a.cap - 1) : a.bt;
    dma4(src, sidx + 64 * r);
  }
}

// Stage B: DMA the block-table entry of every slot into scratch page[].
template <int MODE>
__device__ __forceinline__ void meta_stage_b(const AttnArgs& a, const SeqInfo& si, int b, int wbase, int w1,
                                             int lane, WaveMeta& wm, int nb) {
  const int32_t* sidx = reinterpret_cast<const int32_t*>(wm.vis[nb]);
  int32_t* spg = reinterpret_cast<int32_t*>(wm.vis[nb]) + kMT;
#pragma unroll
  for (int r = 0; r < kTokPerLane; ++r) {
    const int tok = lane + 64 * r;
    int pos, jt;
    uint64_t v;
    slot_pos<MODE>(a, si, wbase, w1, tok, (MODE == MODE_LIST_SHARED) ? sidx[tok] : 0, pos, jt, v);
    if (MODE == MODE_LIST_SHARED && a.phys && jt < 0) continue;   // a listed physical slot needs no lookup
    const int pi = pos >> a.lg_page;
    const bool ok = pos >= 0 && pi < a.max_pages;
    dma4(a.bt + (size_t)b * a.max_pages + (ok ? pi : 0), spg + 64 * r);
  }
}

// Stage C: rows, masks and per-step flags of the window into buffer nb.
template <int MODE>
__device__ __forceinline__ void meta_stage_c(const AttnArgs& a, const SeqInfo& si, int g, int wbase, int w1,
                                             uint64_t colmask, int lane, WaveMeta& wm, int nb) {
  const int P = 1 << a.lg_page;
  const int32_t* sidx = reinterpret_cast<const int32_t*>(wm.vis[nb]);
  const int32_t* spg = sidx + kMT;
  int idx[kTokPerLane], page[kTokPerLane];
#pragma unroll
  for (int r = 0; r < kTokPerLane; ++r) {
    idx[r] = (MODE == MODE_LIST_SHARED) ? sidx[lane + 64 * r] : 0;
    page[r] = spg[lane + 64 * r];
  }
#pragma unroll
  for (int r = 0; r < kTokPerLane; ++r) {
    const int tok = lane + 64 * r;
    int pos, jt;
    uint64_t v;
    slot_pos<MODE>(a, si, wbase, w1, tok, idx[r], pos, jt, v);
    const uint64_t cm = shfl64(colmask, jt & 63);     // every lane takes part in the shuffle
    if (jt >= 0) v = (jt < 64 || a.rowmask == nullptr) ? cm : 0;
    int row = -1;
    if (MODE == MODE_NSA && si.br == BR_CMP) {
      if (pos >= 0) row = si.cbase + pos;        // compressed cache, not paged
    } else if (MODE == MODE_LIST_SHARED && a.phys && jt < 0) {
      const int pg = pos >> a.lg_page;           // a listed entry is a physical slot
      if (pos >= 0 && pg < a.num_pages) row = ((pg * a.Hkv + g) << a.lg_page) | (pos & (P - 1));
    } else if (pos >= 0 && (pos >> a.lg_page) < a.max_pages && (unsigned)page[r] < (unsigned)a.num_pages) {
      row = ((page[r] * a.Hkv + g) << a.lg_page) | (pos & (P - 1));
    }
    if (row < 0) v = 0;
    wm.row[nb][tok] = row;
    wm.vis[nb][tok] = v;
    const uint64_t ok = __ballot(row >= 0 && v == kAll);
    if (lane == 0) {
      wm.full[nb][2 * r] = (uint32_t)ok == 0xffffffffu;
      wm.full[nb][2 * r + 1] = (uint32_t)(ok >> 32) == 0xffffffffu;
    }
  }
}

// DMA the K and V operands of the step described by rows (32 slots) into a ring slot.
// K: each 16-token tile is moved as whole rows (every request a full cache line):
// DMA i of a tile carries 64/RCH consecutive token rows, lane l taking token
// i*(64/RCH) + l/RCH and storing 16-byte chunk p = l % RCH of that row at LDS chunk p;
// it fetches global chunk p ^ (token % RCH), so that the later MFMA-layout reads
// (16 lanes, one chunk index each, 16 different rows) fall on different banks.
// Tile tt occupies blocks [tt*16/(64/RCH), ...) of 1 KB; V: token t -> block KDMA+t.
template <int D, bool NT>
__device__ __forceinline__ void step_dma(const uint16_t* kb, const uint16_t* vb, const int32_t* rows, char* slot,
                                         int lane, int x, int j) {
  constexpr int RCH = D / 8;          // 16-byte chunks per row
  constexpr int RPI = 64 / RCH;       // rows per DMA
  constexpr int IPT = 16 / RPI;       // DMAs per 16-token tile
  const int rq = lane / RCH, p = lane % RCH;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      const int tok = 16 * tt + RPI * i + rq;
      const int c = p ^ (tok % RCH);
      dma16<NT>(kb + (size_t)max(rows[tok], 0) * D + 8 * c, slot + (tt * IPT + i) * 1024);
    }
  const int4 rv0 = *reinterpret_cast<const int4*>(rows + 4 * j);
  const int4 rv1 = *reinterpret_cast<const int4*>(rows + 16 + 4 * j);
  const int rv[8] = {rv0.x, rv0.y, rv0.z, rv0.w, rv1.x, rv1.y, rv1.z, rv1.w};
  const int dx = 8 * (x & (D / 8 - 1));   // d = 64: lanes x >= 8 repeat x - 8 (rows unused)
#pragma unroll
  for (int t = 0; t < 8; ++t) dma16<NT>(vb + (size_t)max(rv[t], 0) * D + dx, slot + (2 * IPT + t) * 1024);
}

// The same DMAs one at a time, so that a refill can be spread through the compute of
// a step: dma_rows reads, for this lane, the cache row of each of the NDMA pieces, and
// dma_piece issues piece n (pieces 0 .. 2*IPT-1 are K, the last 8 are V).
template <int D>
struct DmaGeom {
  static constexpr int RCH = D / 8, RPI = 64 / RCH, IPT = 16 / RPI, NK = 2 * IPT, N = NK + 8;
};
template <int D>
__device__ __forceinline__ void dma_rows(const int32_t* rows, int lane, int j, int (&sr)[DmaGeom<D>::N]) {
  using G = DmaGeom<D>;
  const int rq = lane / G::RCH;
#pragma unroll
  for (int n = 0; n < G::NK; ++n) sr[n] = rows[16 * (n / G::IPT) + G::RPI * (n % G::IPT) + rq];
  const int4 rv0 = *reinterpret_cast<const int4*>(rows + 4 * j);
  const int4 rv1 = *reinterpret_cast<const int4*>(rows + 16 + 4 * j);
  sr[G::NK + 0] = rv0.x; sr[G::NK + 1] = rv0.y; sr[G::NK + 2] = rv0.z; sr[G::NK + 3] = rv0.w;
  sr[G::NK + 4] = rv1.x; sr[G::NK + 5] = rv1.y; sr[G::NK + 6] = rv1.z; sr[G::NK + 7] = rv1.w;
}
template <int D, int n, bool NT>
__device__ __forceinline__ void dma_piece(const uint16_t* kb, const uint16_t* vb, const int (&sr)[DmaGeom<D>::N],
                                          char* slot, int lane, int x) {
  using G = DmaGeom<D>;
  if (n < G::NK) {
    const int tok = 16 * (n / G::IPT) + G::RPI * (n % G::IPT) + lane / G::RCH;
    const int c = (lane % G::RCH) ^ (tok % G::RCH);
    dma16<NT>(kb + (size_t)max(sr[n], 0) * D + 8 * c, slot + n * 1024);
  } else {
    dma16<NT>(vb + (size_t)max(sr[n], 0) * D + 8 * (x & (D / 8 - 1)), slot + n * 1024);
  }
}

// Merge split-K partials in split order.  One wave per q-row.  Lane s loads the
// (m, l) of split s while every lane also loads its columns of the first KC splits
// (KC = 8, 16 or 32: the least that covers n_split, so that a call with few splits
// issues few column loads); later chunks are loaded one chunk ahead of their use, so
// the common case (n_split <= 32) costs one memory round trip.  Split weights reach
// the column loop through readlane.
// q-rows (one wave each) per combine workgroup: few rows per workgroup spread a call's
// rows over more CUs, which shortens the launch's one round trip (measured: a draft
// step's combine 0.75 us faster with one row than with four, verify's 0.6 us with two)
template <int MODE>
constexpr int combine_rows() { return MODE == MODE_DENSE ? 2 : 1; }
constexpr int kChunk = 32;

__device__ __forceinline__ float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Merge the split-K partials of q-row r of pair pid (= (b*Hkv + g)*n_rc + rc) in split
// order and write its output row and lse.  One wave.
template <int D, int KC>
__device__ __forceinline__ void merge_row(const AttnArgs& a, int pid, int r, int lane) {
  const int rc = pid % a.n_rc;
  const int bg = pid / a.n_rc;
  const int g = bg % a.Hkv;
  const int b = bg / a.Hkv;
  const int r0 = rc * kMaxRowsPerWG;
  const int ns = a.n_split;                     // 2 .. kMaxSplits = 128
  const size_t pstride = (size_t)kMaxRowsPerWG * (D + 2);
  const float* base = a.part + (size_t)pid * ns * pstride;
  const float* mcol = base + (size_t)kMaxRowsPerWG * D + r;
  constexpr int CPL = D / 64;                   // columns per lane (2 or 1)
  const float* ocol = base + (size_t)r * D + CPL * lane;
  float cur[KC][CPL], nxt[KC][CPL];
#pragma unroll
  for (int u = 0; u < KC; ++u)
#pragma unroll
    for (int c = 0; c < CPL; ++c) cur[u][c] = ocol[(size_t)min(u, ns - 1) * pstride + c];
  float mv[2], lv[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int sp = lane + 64 * u;
    const size_t o = (size_t)min(sp, ns - 1) * pstride;
    mv[u] = mcol[o];
    lv[u] = mcol[o + kMaxRowsPerWG];
    if (sp >= ns) { mv[u] = -INFINITY; lv[u] = 0.f; }
  }
  const float M = wave_max_f32(fmaxf(mv[0], mv[1]));
  const float Ms = (M == -INFINITY) ? 0.f : M;
  float wv[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) wv[u] = __builtin_amdgcn_exp2f(mv[u] - Ms);
  // butterfly sum: every lane ends with the same, run-to-run fixed value
  const float Ls = wave_sum_f32(wv[0] * lv[0] + wv[1] * lv[1]);
  float acc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
  for (int c0 = 0; c0 < ns; c0 += KC) {
    const bool more = c0 + KC < ns;
    if (more) {
#pragma unroll
      for (int u = 0; u < KC; ++u)
#pragma unroll
        for (int c = 0; c < CPL; ++c) nxt[u][c] = ocol[(size_t)min(c0 + KC + u, ns - 1) * pstride + c];
    }
#pragma unroll
    for (int u = 0; u < KC; ++u) {
      const int sp = c0 + u;
      const float w = (sp < ns) ? lane_f(sp < 64 ? wv[0] : wv[1], sp & 63) : 0.f;
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[c] += w * cur[u][c];
    }
    if (more) {
#pragma unroll
      for (int u = 0; u < KC; ++u)
#pragma unroll
        for (int c = 0; c < CPL; ++c) cur[u][c] = nxt[u][c];
    }
  }
  const float inv = (Ls > 0.f) ? 1.f / Ls : 0.f;
  const int rr = r0 + r;
  const int i = rr / a.G;
  const int h = g * a.G + (rr - i * a.G);
  float* op = a.out + ((size_t)(b * a.n_q + i) * a.Hq + h) * D + CPL * lane;
#pragma unroll
  for (int c = 0; c < CPL; ++c) op[c] = acc[c] * inv;
  if (lane == 0 && a.lse != nullptr)
    a.lse[(size_t)(b * a.n_q + i) * a.Hq + h] = (Ls > 0.f) ? (M + __log2f(Ls)) * kLn2 : -INFINITY;
}

// NSA: merge each branch's splits in split order, then out = sum over branches of gate *
// branch output; lse [B][n_q][Hq][3] holds each branch's log-sum-exp (-inf for a branch
// that saw nothing).  The launch's splits are the compression, selection and window
// branches' in that order.  One pass: lane s loads the (m, l) of split s and every lane
// its columns of all splits (the first KC at once), as in merge_row, and each split
// adds into its own branch's accumulator.
template <int D, int KC>
__device__ __forceinline__ void merge_row_nsa(const AttnArgs& a, int pid, int r, int lane) {
  constexpr int CPL = D / 64;
  const int rc = pid % a.n_rc;
  const int bg = pid / a.n_rc;
  const int g = bg % a.Hkv;
  const int b = bg / a.Hkv;
  const int ns = a.n_split;                     // 3 .. kMaxSplits
  const int e0 = a.ns0, e1 = a.ns0 + a.ns1;     // first selection split, first window split
  const size_t pstride = (size_t)kMaxRowsPerWG * (D + 2);
  const float* base = a.part + (size_t)pid * ns * pstride;
  const float* mcol = base + (size_t)kMaxRowsPerWG * D + r;
  const float* ocol = base + (size_t)r * D + CPL * lane;
  float cur[KC][CPL], nxt[KC][CPL];
#pragma unroll
  for (int u = 0; u < KC; ++u)
#pragma unroll
    for (int c = 0; c < CPL; ++c) cur[u][c] = ocol[(size_t)min(u, ns - 1) * pstride + c];
  float mv[2], lv[2];
  int bv[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int sp = lane + 64 * u;
    const size_t o = (size_t)min(sp, ns - 1) * pstride;
    mv[u] = mcol[o];
    lv[u] = mcol[o + kMaxRowsPerWG];
    bv[u] = (sp >= e1) ? 2 : (sp >= e0 ? 1 : 0);
    if (sp >= ns) { mv[u] = -INFINITY; lv[u] = 0.f; }
  }
  float M[3], Ls[3], wv[2];
#pragma unroll
  for (int br = 0; br < 3; ++br) {
    M[br] = wave_max_f32(fmaxf(bv[0] == br ? mv[0] : -INFINITY, bv[1] == br ? mv[1] : -INFINITY));
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const float Mb = (bv[u] == 0) ? M[0] : (bv[u] == 1 ? M[1] : M[2]);
    wv[u] = __builtin_amdgcn_exp2f(mv[u] - ((Mb == -INFINITY) ? 0.f : Mb));
  }
#pragma unroll
  for (int br = 0; br < 3; ++br) {
    // butterfly sum: every lane ends with the same, run-to-run fixed value
    Ls[br] = wave_sum_f32((bv[0] == br ? wv[0] * lv[0] : 0.f) + (bv[1] == br ? wv[1] * lv[1] : 0.f));
  }
  float acc[3][CPL];
#pragma unroll
  for (int br = 0; br < 3; ++br)
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[br][c] = 0.f;
  for (int c0 = 0; c0 < ns; c0 += KC) {
    const bool more = c0 + KC < ns;
    if (more) {
#pragma unroll
      for (int u = 0; u < KC; ++u)
#pragma unroll
        for (int c = 0; c < CPL; ++c) nxt[u][c] = ocol[(size_t)min(c0 + KC + u, ns - 1) * pstride + c];
    }
#pragma unroll
    for (int u = 0; u < KC; ++u) {
      const int sp = c0 + u;
      if (sp >= ns) break;
      const float w = lane_f(sp < 64 ? wv[0] : wv[1], sp & 63);
      const int br = (sp >= e1) ? 2 : (sp >= e0 ? 1 : 0);
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        if (br == 0) acc[0][c] += w * cur[u][c];
        else if (br == 1) acc[1][c] += w * cur[u][c];
        else acc[2][c] += w * cur[u][c];
      }
    }
    if (more) {
#pragma unroll
      for (int u = 0; u < KC; ++u)
#pragma unroll
        for (int c = 0; c < CPL; ++c) cur[u][c] = nxt[u][c];
    }
  }
  const int rr = rc * kMaxRowsPerWG + r;
  const int i = rr / a.G;
  const int h = g * a.G + (rr - i * a.G);
  const size_t qh = (size_t)(b * a.n_q + i) * a.Hq + h;
  float res[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) res[c] = 0.f;
#pragma unroll
  for (int br = 0; br < 3; ++br) {
    const float gate = a.gates[qh * 3 + br];
    const float f = (Ls[br] > 0.f) ? gate / Ls[br] : 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) res[c] += f * acc[br][c];
    if (lane == 0 && a.lse != nullptr)
      a.lse[qh * 3 + br] = (Ls[br] > 0.f) ? (M[br] + __log2f(Ls[br])) * kLn2 : -INFINITY;
  }
  float* op = a.out + qh * D + CPL * lane;
#pragma unroll
  for (int c = 0; c < CPL; ++c) op[c] = res[c];
}

template <int D, int MODE>
__global__ void __launch_bounds__(256) combine_kernel(AttnArgs a) {
  const int pid = blockIdx.x;                   // (b*Hkv + g)*n_rc + rc
  const int rc = pid % a.n_rc;
  const int nrows = min(kMaxRowsPerWG, a.rows - rc * kMaxRowsPerWG);
  const int r = blockIdx.y * combine_rows<MODE>() + (threadIdx.x >> 6);
  if (r >= nrows) return;
  if constexpr (MODE == MODE_NSA) {
    if (a.n_split <= 8) merge_row_nsa<D, 8>(a, pid, r, threadIdx.x & 63);
    else if (a.n_split <= 16) merge_row_nsa<D, 16>(a, pid, r, threadIdx.x & 63);
    else merge_row_nsa<D, kChunk>(a, pid, r, threadIdx.x & 63);
  } else if (a.n_split <= 8) merge_row<D, 8>(a, pid, r, threadIdx.x & 63);
  else if (a.n_split <= 16) merge_row<D, 16>(a, pid, r, threadIdx.x & 63);
  else merge_row<D, kChunk>(a, pid, r, threadIdx.x & 63);
}

// SC: dense verify that writes per-KV-head partial scores of the two collected rows
// instead of their logits (the selector's per-head sum, done here, 2G times fewer bytes)
template <int D, int QT, int MODE, bool SC = false, bool NT = true>
__global__ void __launch_bounds__(256, 1) attn_kernel(AttnArgs a) {
  constexpr int KS = D / 32;                  // k-steps of the QK^T product
  constexpr int NDMA = DmaGeom<D>::N;         // 16-byte DMAs per lane per step
  constexpr int kSlot = NDMA * 1024;          // ring slot bytes per wave
  constexpr int QCH = D / 8;                  // 16-byte chunks per Q row
  constexpr int kPer = 4 * 8 + 2;             // merge floats per lane per q-tile
  constexpr size_t kQBytes = (size_t)QT * 16 * D * 2;
  constexpr size_t kWaveBytes = sizeof(WaveMeta) + 2 * (size_t)kSlot;
  // Collected logit rows are staged per wave (kStageRows rows x kStageSteps steps) in an
  // area that starts with the Q tile, free once every wave holds Q in registers
  constexpr bool kCanStage = MODE == MODE_DENSE && !SC;
  constexpr size_t kStageWave = (size_t)kStageRows * kStageStride * 4;
  constexpr size_t kHead = (kCanStage && kWaves * kStageWave > kQBytes) ? kWaves * kStageWave : kQBytes;
  constexpr size_t kLoopBytes = kHead + kWaves * kWaveBytes;
  constexpr size_t kMergeBytes = (size_t)kWaves * QT * kPer * 64 * 4;
  constexpr size_t kSmem = kLoopBytes > kMergeBytes ? kLoopBytes : kMergeBytes;
  __shared__ __attribute__((aligned(16))) unsigned char smem_raw[kSmem];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int x = lane & 15;
  const int j = lane >> 4;
  const int s = blockIdx.x;
  const int g = blockIdx.y % a.Hkv;
  const int rc = blockIdx.y / a.Hkv;
  const int b = blockIdx.z;
  const int r0 = rc * kMaxRowsPerWG;
  const int nrows = min(kMaxRowsPerWG, a.rows - r0);

  uint16_t* s_q = reinterpret_cast<uint16_t*>(smem_raw);
  unsigned char* wbase_lds = smem_raw + kHead + (size_t)wave * kWaveBytes;
  WaveMeta& wm = *reinterpret_cast<WaveMeta*>(wbase_lds);
  char* ring = reinterpret_cast<char*>(wbase_lds + sizeof(WaveMeta));
  float* s_merge = reinterpret_cast<float*>(smem_raw);

  // NSA: the launch's splits are the compression, then selection, then window branch's
  int br = 0, s_loc = s, ns_loc = a.n_split;
  if constexpr (MODE == MODE_NSA) {
    br = (s >= a.ns0 + a.ns1) ? BR_WIN : (s >= a.ns0 ? BR_SLC : BR_CMP);
    s_loc = s - (br == BR_WIN ? a.ns0 + a.ns1 : (br == BR_SLC ? a.ns0 : 0));
    ns_loc = (br == BR_WIN) ? a.ns2 : (br == BR_SLC ? a.ns1 : a.ns0);
  }
  const uint16_t* kb = (MODE == MODE_NSA && br == BR_CMP) ? a.ck : a.k;
  const uint16_t* vb = (MODE == MODE_NSA && br == BR_CMP) ? a.cv : a.v;
  const SeqInfo si = seq_info<MODE>(a, b, g, br);
  // balanced contiguous step ranges: the n_split * kWaves waves of this (sequence, KV
  // head) split its steps evenly (to within one step); a workgroup's waves are adjacent
  // Token-list modes split the launch's step bound (cap + max tail) instead of the
  // sequence's own, so that the index-list DMA can go out before the sequence's counts
  // arrive; waves past the sequence's end then have nothing to do.
  const long long nwv = (long long)ns_loc * kWaves;
  const long long gwv = (long long)s_loc * kWaves + wave;
  const long long Tsp = (MODE == MODE_LIST_SHARED) ? (long long)a.T_max : (long long)si.T;
  const int w0 = (int)(gwv * Tsp / nwv);
  const int w1s = (int)((gwv + 1) * Tsp / nwv);
  const int w1 = min(w1s, si.T);

  // Column mask of verifier/tail slot `lane`: bit i = row i sees that slot.
  uint64_t colmask;
  if (a.rowmask != nullptr) {
    colmask = 0;
    const uint64_t* rm = a.rowmask + (size_t)b * a.n_q;
    for (int i = 0; i < a.n_q; ++i) colmask |= ((rm[i] >> lane) & 1ull) << i;
  } else {
    colmask = (MODE == MODE_DENSE) ? (kAll << lane) : kAll;
  }

  // verifier row index of this lane's q-row in each tile (64 = padding row), and the
  // logit slot of that row (-1: not collected)
  int rowi[QT], cslot[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int r = 16 * qt + x;
    rowi[qt] = (r < nrows) ? (r0 + r) / a.G : 64;
    cslot[qt] = -1;
    if (rowi[qt] < 64 && ((a.cmask >> rowi[qt]) & 1ull))
      cslot[qt] = __popcll(a.cmask & ((1ull << rowi[qt]) - 1)) ^ a.cswap;
  }
  const bool collect = MODE == MODE_DENSE && !SC && a.logits != nullptr;
  // stage the collected rows of kStageSteps steps in LDS and write each row as one run:
  // needs at most kStageRows rows per group and 16-byte aligned rows
  const bool stage = kCanStage && collect && a.lvec4 && a.n_cl * a.G <= kStageRows;

  float m[QT], l[QT];
  f32x4 O[QT][8];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    m[qt] = -INFINITY;
    l[qt] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) O[qt][e] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // Prologue: window-0 metadata DMAs go out together with the Q loads, so the block-table
  // round trip overlaps the Q fetch and the Q -> LDS copy.
  // Physical-slot lists need block-table entries for the tail slots only, whose
  // positions do not depend on the list: those go out together with the list DMA.
  if (MODE == MODE_LIST_SHARED) {
    if (w0 < w1s) meta_stage_a<MODE>(a, si, w0, lane, wm, 0);
    if (a.phys && w0 < w1) meta_stage_b<MODE>(a, si, b, w0, w1, lane, wm, 0);
  } else if (w0 < w1) {
    meta_stage_b<MODE>(a, si, b, w0, w1, lane, wm, 0);
  }
  // Q rows of this workgroup: 16-byte chunk c of row r goes to LDS chunk c ^ (r % QCH)
  constexpr int kQPer = (QT * 16 * QCH + 255) / 256;
  u32x4 qv[kQPer];
#pragma unroll
  for (int u = 0; u < kQPer; ++u) {
    const int e = tid + 256 * u;
    const int r = e / QCH;
    const int c = e - r * QCH;
    qv[u] = u32x4{0, 0, 0, 0};
    if (e < QT * 16 * QCH && r < nrows) {
      const int rr = r0 + r;
      const int i = rr / a.G;
      const int h = g * a.G + (rr - i * a.G);
      qv[u] = *reinterpret_cast<const u32x4*>(a.q + ((size_t)(b * a.n_q + i) * a.Hq + h) * D + 8 * c);
    }
  }
  wait_vm<0>();
  if (MODE == MODE_LIST_SHARED && !a.phys && w0 < w1) meta_stage_b<MODE>(a, si, b, w0, w1, lane, wm, 0);
#pragma unroll
  for (int u = 0; u < kQPer; ++u) {
    const int e = tid + 256 * u;
    const int r = e / QCH;
    const int c = e - r * QCH;
    if (e < QT * 16 * QCH) *reinterpret_cast<u32x4*>(s_q + (r * QCH + (c ^ (r % QCH))) * 8) = qv[u];
  }
  // dense and block modes have the first window's block-table entries already: their
  // first two K/V steps go out before the Q barrier, so the Q staging overlaps them
  if ((MODE != MODE_LIST_SHARED || a.phys) && w0 < w1) {
    meta_stage_c<MODE>(a, si, g, w0, w1, colmask, lane, wm, 0);
    wait_lgkm0();
    step_dma<D, NT>(kb, vb, wm.row[0], ring, lane, x, j);
    if (w0 + 1 < w1) step_dma<D, NT>(kb, vb, wm.row[0] + kStepTokens, ring + kSlot, lane, x, j);
  }
  // Q in LDS.  An LDS-only barrier: __syncthreads would also wait for those DMAs.
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  // Q^T B-operands of this lane (q-row x of each tile, 8 dims per k-step), kept in registers
  u32x4 qop[QT][KS];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int r = 16 * qt + x;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c = 4 * ks + j;
      qop[qt][ks] = *reinterpret_cast<const u32x4*>(s_q + (r * QCH + (c ^ (r % QCH))) * 8);
    }
  }
  // partial scores and staged logit rows use the Q area, free once every wave holds Q
  if (SC || stage) {
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }

  if (w0 < w1) {
    if (MODE == MODE_LIST_SHARED && !a.phys) {
      wait_vm<0>();
      meta_stage_c<MODE>(a, si, g, w0, w1, colmask, lane, wm, 0);
      wait_lgkm0();
      step_dma<D, NT>(kb, vb, wm.row[0], ring, lane, x, j);
      if (w0 + 1 < w1) step_dma<D, NT>(kb, vb, wm.row[0] + kStepTokens, ring + kSlot, lane, x, j);
    }
    // Software pipeline.  Iteration s waits for slot s and moves it to registers, issues
    // the metadata stage, runs S(s) on the matrix core, stores S(s)'s collected logits,
    // and refills slot s with step s+2 (stores count in vmcnt, so they must precede the
    // batch that the next wait leaves outstanding).  Both ring slots are then in flight
    // while one straight-line block runs PV(s-1) from the previous iteration's registers
    // on the matrix core and softmax(s) on the VALU, interleaved by the scheduler.  A
    // rescale decided by softmax(s) is applied to O right after that block, once PV(s-1)
    // is in, so that PV(s) in the next iteration adds to O on the new reference.
    u32x4 vprev[8], phi[QT], plo[QT];
#pragma unroll
    for (int t = 0; t < 8; ++t) vprev[t] = u32x4{0, 0, 0, 0};
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) phi[qt] = plo[qt] = u32x4{0, 0, 0, 0};
    f32x4 S[2][QT];   // S^T of the current step
    float alpha[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) alpha[qt] = 1.f;
    bool pend = false;
    const float c2 = a.scale_log2;

    // O^T += V^T(s-1) P^T(s-1), one transposed V tile at a time; hook(e) runs after tile e
    auto pv = [&](auto hook) {
      static_for<0, 8>([&](auto ec) {
        constexpr int e = decltype(ec)::value;
        u32x4 vte;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t w0v = vprev[2 * w][e >> 1], w1v = vprev[2 * w + 1][e >> 1];
          // even e: low halves of (w0v, w1v); odd e: high halves
          vte[w] = __builtin_amdgcn_perm(w1v, w0v, (e & 1) ? 0x07060302u : 0x05040100u);
        }
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          O[qt][e] = mfma16(vte, phi[qt], O[qt][e]);
          O[qt][e] = mfma16(vte, plo[qt], O[qt][e]);
        }
        hook(ec);
      });
    };
    auto rescale = [&]() {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int e = 0; e < 8; ++e) O[qt][e] *= alpha[qt];
    };
    // Collected rows (Collect-2-Query and its generalisation to any row set): scaled
    // logits, prefix columns only
    auto store_logits = [&](int st) {
      const int p0 = st * kStepTokens + 4 * j;
      const bool whole = a.lvec4 && st * kStepTokens + kStepTokens <= si.L;
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const bool mine = cslot[qt] >= 0;
        if (!__any(mine)) continue;
        const int rr = r0 + 16 * qt + x;
        const int h = g * a.G + (rr - rowi[qt] * a.G);
        float* base = a.logits + ((size_t)(b * a.Hq + h) * a.n_cl + max(cslot[qt], 0)) * a.logits_ld + p0;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          if (!mine || (c == 1 && !a.cdup)) continue;
          float* dst = base + c * a.logits_ld;
          if (whole) {
            // device-scope stores, as for the staged runs (all 9 rows collected at 32K:
            // 48.9 -> 47.6 us against non-temporal stores; 128K x 8: 1126 -> 1111 us)
            store_dev_scope(dst, S[0][qt] * a.scale);
            store_dev_scope(dst + 16, S[1][qt] * a.scale);
          } else {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if (p0 + 16 * tt + i < si.L) dst[16 * tt + i] = S[tt][qt][i] * a.scale;
          }
        }
      }
    };
    // Staged collected rows: each step's scaled logits go to this wave's staging area as
    // [slot c * G + head][kStageStride] (kStageSteps * 32 tokens, then padding); after
    // kStageSteps steps (or the wave's last prefix step) the staged run of every row is
    // written with 16-byte device-scope stores, one row run of up to 512 contiguous
    // bytes per 32 lanes.
    float* stg = reinterpret_cast<float*>(smem_raw) + (size_t)wave * (kStageWave / 4);
    const int st_last = min(w1, (si.L + kStepTokens - 1) / kStepTokens) - 1;   // last prefix step
    int st_first = w0;                                                       // first staged step
    // staged rows that this workgroup's row chunk holds (a row chunk may hold one slot only)
    uint32_t smask = 0;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      if (cslot[qt] < 0) continue;
      const int hh = r0 + 16 * qt + x - rowi[qt] * a.G;
      smask |= 1u << (cslot[qt] * a.G + hh);
      if (a.cdup) smask |= 1u << ((cslot[qt] + 1) * a.G + hh);
    }
    smask = wave_or_u32(smask);
    auto stage_logits = [&](int st) {
      if (st > st_last) return;
      const int col = (st - st_first) * kStepTokens + 4 * j;
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        if (cslot[qt] < 0) continue;
        const int hh = r0 + 16 * qt + x - rowi[qt] * a.G;
        float* dst = stg + (cslot[qt] * a.G + hh) * kStageStride + col;
        *reinterpret_cast<f32x4*>(dst) = S[0][qt] * a.scale;
        *reinterpret_cast<f32x4*>(dst + 16) = S[1][qt] * a.scale;
        if (a.cdup) {
          float* d2 = dst + a.G * kStageStride;
          *reinterpret_cast<f32x4*>(d2) = S[0][qt] * a.scale;
          *reinterpret_cast<f32x4*>(d2 + 16) = S[1][qt] * a.scale;
        }
      }
      if (st - st_first + 1 < kStageSteps && st < st_last) return;
      // flush: chunk q = lane + 64u covers row q / 32 (of n_cl * G rows), 16 bytes at column
      // 4 * (q % 32) of the staged run [st_first * 32, (st + 1) * 32) clipped to the prefix
      wait_lgkm0();
      const int p0 = st_first * kStepTokens;
      const int ncol = min((st + 1) * kStepTokens, si.L) - p0;
      const int nrow = a.n_cl * a.G;
#pragma unroll 1
      for (int u = 0; u < kStageRows * kStageSteps * kStepTokens / 4 / 64; ++u) {
        const int q = lane + 64 * u;
        const int rr = q / (kStageSteps * kStepTokens / 4);
        const int cc = 4 * (q % (kStageSteps * kStepTokens / 4));
        if (rr >= nrow || cc >= ncol || !((smask >> rr) & 1u)) continue;
        const int c = rr / a.G;
        const int h = g * a.G + (rr - c * a.G);
        const f32x4 v = *reinterpret_cast<const f32x4*>(stg + rr * kStageStride + cc);
        float* dst = a.logits + ((size_t)(b * a.Hq + h) * a.n_cl + c) * a.logits_ld + p0 + cc;
        if (cc + 4 <= ncol) {
          store_dev_scope(dst, v);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (cc + e < ncol) dst[e] = v[e];
        }
      }
      st_first = st + 1;
    };
    // Partial scores: the lanes of the collected rows put their scaled logits of the
    // step in this wave's part of the Q area as [slot c * G + head][32 tokens]; lanes
    // 0-31 then sum one token's column over the group's heads, ascending, as
    // acc = acc + (row0 + row1), and store 32 consecutive scores.
    auto store_scores = [&](int st) {
      float* sb = reinterpret_cast<float*>(smem_raw) + (size_t)wave * (kQBytes / 4 / kWaves);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const bool mine = cslot[qt] >= 0;
        if (!__any(mine)) continue;
        if (mine) {
          const int hh = r0 + 16 * qt + x - rowi[qt] * a.G;
          float* dst = sb + (cslot[qt] * a.G + hh) * kStepTokens + 4 * j;
          *reinterpret_cast<f32x4*>(dst) = S[0][qt] * a.scale;
          *reinterpret_cast<f32x4*>(dst + 16) = S[1][qt] * a.scale;
          if (a.cdup) {
            *reinterpret_cast<f32x4*>(dst + a.G * kStepTokens) = S[0][qt] * a.scale;
            *reinterpret_cast<f32x4*>(dst + a.G * kStepTokens + 16) = S[1][qt] * a.scale;
          }
        }
      }
      const int p = st * kStepTokens + lane;
      if (lane < kStepTokens && p < si.L) {
        float acc = 0.f;
        for (int hh = 0; hh < a.G; ++hh) acc = acc + (sb[hh * kStepTokens + lane] + sb[(a.G + hh) * kStepTokens + lane]);
        a.scores[(size_t)(b * a.Hkv + g) * a.scores_ld + p] = acc;
      }
    };
    // PV(s-1) and softmax(s).  The reference max m only moves when a row's max grows
    // by more than 2^kTau, so the O rescale (AGPR round trips) is rare; weights stay
    // below 2^kTau.  P goes out as bf16 hi + lo B-operands.
    // The refill DMAs of the next-but-one step are spread over the PV tiles, so that
    // their issue, which stalls while the memory pipeline is busy, overlaps compute.
    // FAST: every token of the step is visible to every row and a refill is due.
    auto block = [&](const uint64_t* vr, const int (&sr)[NDMA], char* slot, bool dma_due, auto fastc) {
      constexpr bool FAST = decltype(fastc)::value;
      pv([&](auto ec) {
        constexpr int e = decltype(ec)::value;
        static_for<e * NDMA / 8, (e + 1) * NDMA / 8>([&](auto nc) {
          if (FAST || dma_due) dma_piece<D, decltype(nc)::value, NT>(kb, vb, sr, slot, lane, x);
        });
      });
      bool grow_any = false;
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        float t8[8];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i) t8[4 * tt + i] = S[tt][qt][i];
        if (!FAST) {
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (((vr[16 * tt + 4 * j + i] >> rowi[qt]) & 1ull) == 0) t8[4 * tt + i] = -INFINITY;
        }
        const float rmax = colmax4(max3f(max3f(t8[0], t8[1], t8[2]), max3f(t8[3], t8[4], t8[5]),
                                         max3f(t8[6], t8[7], t8[7])));
        const float mx = rmax * c2;
        const bool grow = mx > m[qt] + kTau;
        // rows that keep their reference (possibly still -inf) keep alpha = 1
        alpha[qt] = grow ? __builtin_amdgcn_exp2f(m[qt] - mx) : 1.f;
        m[qt] = grow ? mx : m[qt];
        grow_any = grow_any || grow;
        const float nms = (m[qt] == -INFINITY) ? 0.f : -m[qt];
        float psum = 0.f;
#pragma unroll
        for (int u = 0; u < 8; u += 2) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(t8[u], c2, nms));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(t8[u + 1], c2, nms));
          psum += p0 + p1;
          const uint32_t hw = pack_bf16(p0, p1);
          phi[qt][u >> 1] = hw;
          plo[qt][u >> 1] = pack_bf16(p0 - __uint_as_float(hw << 16), p1 - __uint_as_float(hw & 0xffff0000u));
        }
        l[qt] = l[qt] * alpha[qt] + psum;
      }
      pend = __any(grow_any);
    };

    for (int wb = w0, k = 0; wb < w1; wb += kMW, ++k) {
      const int buf = k & 1;
      const bool next_win = wb + kMW < w1;
      const int nloc = min(kMW, w1 - wb);
      for (int ls = 0; ls < nloc; ++ls) {
        const int step = wb + ls;
        char* slot = ring + ((step - w0) & 1) * kSlot;
        // this step's DMAs are done once at most one step's worth is outstanding
        if (step + 1 < w1) wait_vm<NDMA>();
        else wait_vm<0>();
        u32x4 kop[2][KS], vcur[8];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int kpos = ((4 * ks + j) ^ (x % QCH)) * 16;   // swizzled chunk of row x
          kop[0][ks] = *reinterpret_cast<const u32x4*>(slot + x * (2 * D) + kpos);
          kop[1][ks] = *reinterpret_cast<const u32x4*>(slot + (16 + x) * (2 * D) + kpos);
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) vcur[t] = *reinterpret_cast<const u32x4*>(slot + (2 * KS + t) * 1024 + 16 * lane);
        const bool full = wm.full[buf][ls] != 0;
        if (!full) {
          // invalid slots were loaded from row 0: zero them, since a masked weight
          // times a NaN in an unused cache slot would still poison O
          const int32_t* rows = wm.row[buf] + ls * kStepTokens;
          const int4 rv0 = *reinterpret_cast<const int4*>(rows + 4 * j);
          const int4 rv1 = *reinterpret_cast<const int4*>(rows + 16 + 4 * j);
          const int rv[8] = {rv0.x, rv0.y, rv0.z, rv0.w, rv1.x, rv1.y, rv1.z, rv1.w};
#pragma unroll
          for (int t = 0; t < 8; ++t)
            if (rv[t] < 0) vcur[t] = u32x4{0, 0, 0, 0};
        }
        wait_lgkm0();   // the slot is in registers: it may be refilled
        // next window's metadata, one stage per step
        if (next_win) {
          if (ls == 0) meta_stage_a<MODE>(a, si, wb + kMW, lane, wm, buf ^ 1);
          if (ls == 1) meta_stage_b<MODE>(a, si, b, wb + kMW, w1, lane, wm, buf ^ 1);
          if (ls == 2) meta_stage_c<MODE>(a, si, g, wb + kMW, w1, colmask, lane, wm, buf ^ 1);
        }
        // S^T(s) = K Q^T for two 16-token tiles
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          S[0][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
          S[1][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            S[0][qt] = mfma16(kop[0][ks], qop[qt][ks], S[0][qt]);
            S[1][qt] = mfma16(kop[1][ks], qop[qt][ks], S[1][qt]);
          }
        }
        if (stage) stage_logits(step);
        else if (collect) store_logits(step);
        if constexpr (SC) store_scores(step);
        // cache rows of step s+2, which refills this slot (read even when no refill is
        // due: the pointer stays inside this wave's metadata area)
        const bool dma_due = step + 2 < w1;
        int sr[NDMA];
        {
          const int ns = ls + 2;
          dma_rows<D>((ns < kMW) ? wm.row[buf] + ns * kStepTokens : wm.row[buf ^ 1] + (ns - kMW) * kStepTokens,
                      lane, j, sr);
        }
        if (full && dma_due) block(nullptr, sr, slot, true, std::true_type{});
        else block(wm.vis[buf] + ls * kStepTokens, sr, slot, dma_due, std::false_type{});
        if (pend) rescale();
#pragma unroll
        for (int t = 0; t < 8; ++t) vprev[t] = vcur[t];
      }
    }
    // drain: PV of the last step
    pv([](auto) {});
  }

  // full row sums (fixed order)
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) l[qt] = sum_x16_x32(l[qt]);

  // ---- merge the 4 waves' states through LDS.  Every wave publishes (m, l, O); then
  //      wave w merges dims {8i + 2w, 8i + 2w + 1} of every row, in wave order 0..3.
  __syncthreads();   // every wave is done with Q, its metadata and its ring
  {
    // O tile e of a lane as one 16-byte store: floats [(qt * kPer + 4 e) * 64, + 256) hold
    // the tile's four values of every lane, lane-major
    float* w = s_merge + (size_t)wave * QT * kPer * 64;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *reinterpret_cast<f32x4*>(w + (qt * kPer + e * 4) * 64 + 4 * lane) = O[qt][e];
      w[(qt * kPer + 32) * 64 + lane] = m[qt];
      w[(qt * kPer + 33) * 64 + lane] = l[qt];
    }
  }
  __syncthreads();
  const int e0 = 2 * wave;          // this wave's two O tiles (dims 32j + 8i + e0 + {0, 1})
  float mo[QT], lo_[QT], oo[QT][2][4];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    float M = -INFINITY;
#pragma unroll
    for (int ow = 0; ow < kWaves; ++ow) M = fmax2(M, s_merge[((size_t)ow * QT * kPer + qt * kPer + 32) * 64 + lane]);
    const float Ms = (M == -INFINITY) ? 0.f : M;
    float L = 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) oo[qt][h][i] = 0.f;
#pragma unroll
    for (int ow = 0; ow < kWaves; ++ow) {
      const float* w = s_merge + (size_t)ow * QT * kPer * 64;
      const float mw = w[(qt * kPer + 32) * 64 + lane];
      const float sc = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - Ms);
      L += sc * w[(qt * kPer + 33) * 64 + lane];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const f32x4 t = *reinterpret_cast<const f32x4*>(w + (qt * kPer + (e0 + h) * 4) * 64 + 4 * lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) oo[qt][h][i] += sc * t[i];
      }
    }
    mo[qt] = M;
    lo_[qt] = L;
  }

  // ---- write: lane (x, j) holds q-row x, dims 32j + 8i + e0 + {0,1} (i < 4); for d = 64
  //      only j < 2 holds real dims.  Final output with one split, else a partial.
  const size_t pstride = (size_t)kMaxRowsPerWG * (D + 2);
  const int pid = (b * a.Hkv + g) * a.n_rc + rc;
  const size_t pidx = (size_t)pid * a.n_split + s;
  const int d0 = 32 * j + e0;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int r = 16 * qt + x;
    if (r >= nrows || 32 * j >= D) continue;
    if (MODE != MODE_NSA && a.n_split == 1) {
      const int rr = r0 + r;
      const int i = rr / a.G;
      const int h = g * a.G + (rr - i * a.G);
      const float inv = (lo_[qt] > 0.f) ? 1.f / lo_[qt] : 0.f;
      float* op = a.out + ((size_t)(b * a.n_q + i) * a.Hq + h) * D + d0;
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        *reinterpret_cast<float2*>(op + 8 * i4) = make_float2(oo[qt][0][i4] * inv, oo[qt][1][i4] * inv);
      if (wave == 0 && j == 0 && a.lse != nullptr)
        a.lse[(size_t)(b * a.n_q + i) * a.Hq + h] =
            (lo_[qt] > 0.f) ? (mo[qt] + __log2f(lo_[qt])) * kLn2 : -INFINITY;
    } else {
      float* pp = a.part + pidx * pstride;
      float* op = pp + (size_t)r * D + d0;
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        *reinterpret_cast<float2*>(op + 8 * i4) = make_float2(oo[qt][0][i4], oo[qt][1][i4]);
      if (wave == 0 && j == 0) {
        pp[(size_t)kMaxRowsPerWG * D + r] = mo[qt];
        pp[(size_t)kMaxRowsPerWG * D + kMaxRowsPerWG + r] = lo_[qt];
      }
    }
  }
}

// Union of the n_q rows' block lists of one (b, g), ascending, with per-block row masks
// (SSV page, section 4.2: shared blocks are scheduled once for the whole group).
constexpr int kPlanChunk = 4096;

__global__ void __launch_bounds__(256) block_union_kernel(AttnArgs a) {
  const int bg = blockIdx.x;
  const int g = bg % a.Hkv;
  const int b = bg / a.Hkv;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  __shared__ uint32_t mlo[kPlanChunk];
  __shared__ uint32_t mhi[kPlanChunk];
  __shared__ uint32_t wsum[4];
  __shared__ int32_t scnt[64];
  int32_t* ub = const_cast<int32_t*>(a.ublk) + (size_t)bg * a.ucap;
  uint64_t* um = const_cast<uint64_t*>(a.umask) + (size_t)bg * a.ucap;
  const uint64_t all_rows = (a.n_q >= 64) ? kAll : ((1ull << a.n_q) - 1);
  int total = 0;
  for (int base = 0; base < a.max_pages; base += kPlanChunk) {
    const int span = min(kPlanChunk, a.max_pages - base);     // block ids of this chunk
    for (int e = tid; e < span; e += 256) mlo[e] = mhi[e] = 0;
    __syncthreads();
    // every (row, entry) pair at once, so that the list loads do not wait on each other
    if (tid < a.n_q) scnt[tid] = min(max(a.counts[(size_t)(b * a.n_q + tid) * a.Hkv + g], 0), a.cap);
    __syncthreads();
    const int n_ent = a.n_q * a.cap;
    for (int f = tid; f < n_ent; f += 256) {
      const int i = f / a.cap, e = f - i * a.cap;
      if (e >= scnt[i]) continue;
      const int blk = a.indices[((size_t)(b * a.n_q + i) * a.Hkv + g) * a.cap + e];
      if (blk >= base && blk < base + span) {
        if (i < 32) atomicOr(&mlo[blk - base], 1u << i);
        else atomicOr(&mhi[blk - base], 1u << (i - 32));
      }
    }
    __syncthreads();
    // ascending compaction: thread t owns ids [16t, 16t + 16) of the chunk; an exclusive
    // scan of the per-thread counts (wave scan, then the four wave totals)
    uint32_t c = 0;
    for (int e = 0; e < 16; ++e) {
      const int id = 16 * tid + e;
      c += (id < span) && ((mlo[id] | mhi[id]) != 0);
    }
    const uint32_t x = wave_incl_scan(c);
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    uint32_t pre = 0, chunk_total = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pre += (i < w) ? wsum[i] : 0u;
      chunk_total += wsum[i];
    }
    uint32_t pos = total + pre + x - c;
    for (int e = 0; e < 16; ++e) {
      const int id = 16 * tid + e;
      if (id >= span) break;
      const uint64_t msk = ((uint64_t)mhi[id] << 32) | mlo[id];
      if (msk != 0 && (int)pos < a.ucap) {
        ub[pos] = base + id;
        um[pos] = a.approx ? all_rows : msk;   // approximate: every row sees the union
        ++pos;
      }
    }
    total += chunk_total;
    __syncthreads();
  }
  if (tid == 0) const_cast<int32_t*>(a.ucount)[bg] = min(total, a.ucap);
}

// NSA token compression: compressed row i of (b, g) is the mean of the K (V) rows of
// positions [i*stride, i*stride + len), rounded to bf16 (nearest, ties to even); rows of
// blocks that do not lie entirely in the prefix are zero.  Lane group: one compressed row,
// one 16-byte chunk of dims per lane; the len rows are summed in position order in fp32.
template <int D>
__global__ void __launch_bounds__(256) compress_kernel(AttnArgs a, const int32_t* prefix_len, uint16_t* kc,
                                                       uint16_t* vc) {
  constexpr int CH = D / 8;           // 16-byte chunks per row
  constexpr int RPW = 256 / CH;       // compressed rows per workgroup
  constexpr int kPgCap = 512;         // block-table entries staged in LDS per workgroup
  constexpr int kBatch = 8;           // tokens whose K and V loads go out together
  __shared__ int32_t s_pg[kPgCap];
  const int g = blockIdx.y, b = blockIdx.z;
  const int i_base = blockIdx.x * RPW;
  const int i = i_base + (int)threadIdx.x / CH;
  const int c = (int)threadIdx.x % CH;
  if (i_base >= a.max_cmp) return;
  const int P = 1 << a.lg_page;
  const int L = min(max(prefix_len[b], 0), a.max_prefix_len);
  const int n = (L < a.cmp_len) ? 0 : min((L - a.cmp_len) / a.cmp_stride + 1, a.max_cmp);
  const int32_t* bt = a.bt + (size_t)b * a.max_pages;
  // the block-table entries of the workgroup's token span go to LDS in one round trip,
  // so that every token's K and V loads can go out without waiting on its page
  const int i_last = min(i_base + RPW, n) - 1;
  const int pg0 = (i_base * a.cmp_stride) >> a.lg_page;
  const int npg = (i_last >= i_base) ? ((i_last * a.cmp_stride + a.cmp_len - 1) >> a.lg_page) - pg0 + 1 : 0;
  const bool staged = npg <= kPgCap;
  if (staged)
    for (int e = threadIdx.x; e < npg; e += 256) s_pg[e] = bt[pg0 + e];
  __syncthreads();
  u32x4 ko = u32x4{0, 0, 0, 0}, vo = u32x4{0, 0, 0, 0};
  if (i < n) {
    float ks[8], vs[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) ks[e] = vs[e] = 0.f;
    const int p0 = i * a.cmp_stride;
    for (int t0 = 0; t0 < a.cmp_len; t0 += kBatch) {
      u32x4 kk[kBatch], vv[kBatch];
      bool ok[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int p = p0 + t0 + u;
        int page = -1;
        if (t0 + u < a.cmp_len) page = staged ? s_pg[(p >> a.lg_page) - pg0] : bt[p >> a.lg_page];
        ok[u] = (unsigned)page < (unsigned)a.num_pages;   // outside the cache: skipped
        // a skipped token loads row 0 (always in bounds) and is not added
        const size_t row = ok[u] ? (((size_t)(page * a.Hkv + g) << a.lg_page) | (size_t)(p & (P - 1))) : 0;
        kk[u] = *reinterpret_cast<const u32x4*>(a.k + row * D + 8 * c);
        vv[u] = *reinterpret_cast<const u32x4*>(a.v + row * D + 8 * c);
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (!ok[u]) continue;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          ks[2 * w] += bf16_to_f32(kk[u][w] & 0xffffu);
          ks[2 * w + 1] += bf16_to_f32(kk[u][w] >> 16);
          vs[2 * w] += bf16_to_f32(vv[u][w] & 0xffffu);
          vs[2 * w + 1] += bf16_to_f32(vv[u][w] >> 16);
        }
      }
    }
    const float inv = 1.f / (float)a.cmp_len;     // a power of two: exact
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      ko[w] = pack_bf16(ks[2 * w] * inv, ks[2 * w + 1] * inv);
      vo[w] = pack_bf16(vs[2 * w] * inv, vs[2 * w + 1] * inv);
    }
  }
  if (i >= a.max_cmp) return;
  const size_t o = ((size_t)(b * a.Hkv + g) * a.max_cmp + i) * D + 8 * c;
  *reinterpret_cast<u32x4*>(kc + o) = ko;
  *reinterpret_cast<u32x4*>(vc + o) = vo;
}

template <int D, int MODE>
hipError_t launch_main_mode(const AttnPlan& p, const AttnArgs& a, hipStream_t stream) {
  dim3 grid(p.n_split, a.Hkv * p.n_rc, a.B);
  bool launched = false;
  if constexpr (MODE == MODE_DENSE) {
    if (a.scores != nullptr) {
      switch (p.QT) {
        case 1: hipLaunchKernelGGL((attn_kernel<D, 1, MODE, true>), grid, dim3(256), 0, stream, a); break;
        case 2: hipLaunchKernelGGL((attn_kernel<D, 2, MODE, true>), grid, dim3(256), 0, stream, a); break;
        default: hipLaunchKernelGGL((attn_kernel<D, 3, MODE, true>), grid, dim3(256), 0, stream, a); break;
      }
      launched = true;
    }
  }
  if (!launched) switch (p.QT) {
    case 1: hipLaunchKernelGGL((attn_kernel<D, 1, MODE>), grid, dim3(256), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((attn_kernel<D, 2, MODE>), grid, dim3(256), 0, stream, a); break;
    default:   // several row chunks re-read the same K/V: cached loads
      if (p.n_rc > 1) hipLaunchKernelGGL((attn_kernel<D, 3, MODE, false, false>), grid, dim3(256), 0, stream, a);
      else hipLaunchKernelGGL((attn_kernel<D, 3, MODE>), grid, dim3(256), 0, stream, a);
      break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || (MODE != MODE_NSA && p.n_split == 1)) return e;
  const int rows_wg = p.rows < kMaxRowsPerWG ? p.rows : kMaxRowsPerWG;
  constexpr int CR = combine_rows<MODE>();
  hipLaunchKernelGGL((combine_kernel<D, MODE>), dim3(a.B * a.Hkv * p.n_rc, (rows_wg + CR - 1) / CR),
                     dim3(64 * CR), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_main(const AttnPlan& p, const AttnArgs& a, hipStream_t stream) {
  // the two token-list modes differ only in which list a KV head reads
  if (a.mode == MODE_DENSE) return launch_main_mode<D, MODE_DENSE>(p, a, stream);
  if (a.mode == MODE_BLOCK) return launch_main_mode<D, MODE_BLOCK>(p, a, stream);
  if (a.mode == MODE_NSA) return launch_main_mode<D, MODE_NSA>(p, a, stream);
  return launch_main_mode<D, MODE_LIST_SHARED>(p, a, stream);
}

}  // namespace

AttnPlan attn_plan(int32_t mode, int32_t B, int32_t n_q, int32_t Hq, int32_t Hkv, int32_t d,
                   int32_t page_size, int32_t max_prefix_len, int32_t cap, int32_t max_tail_len,
                   int32_t cus) {
  AttnPlan p{};
  const long long ncu = cus > 0 ? cus : kDefaultCUs;
  p.D = d;
  const int G = Hq / Hkv;
  p.rows = n_q * G;
  p.n_rc = (p.rows + kMaxRowsPerWG - 1) / kMaxRowsPerWG;
  const int rows_wg = p.rows < kMaxRowsPerWG ? p.rows : kMaxRowsPerWG;
  p.QT = (rows_wg + 15) / 16;
  long long T;
  if (mode == MODE_DENSE) {
    T = ((long long)max_prefix_len + n_q + kStepTokens - 1) / kStepTokens;
  } else if (mode == MODE_BLOCK) {
    T = (long long)n_q * cap * (page_size / kStepTokens) + (max_tail_len + kStepTokens - 1) / kStepTokens;
  } else {
    T = ((long long)cap + max_tail_len + kStepTokens - 1) / kStepTokens;
  }
  if (T < 1) T = 1;
  p.T_max = (int32_t)T;
  long long pairs = (long long)B * Hkv * p.n_rc;
  if (pairs < 1) pairs = 1;
  // Token lists: one round of workgroups, one per CU.  The start-up chain of dependent
  // loads (sequence bounds, index list, block table) is paid once per workgroup, so
  // fewer, longer workgroups stream more of the time.  Dense verify: four rounds, which
  // measured ~5% faster at 128K x 8 (each round covers fewer sequences at once).  A
  // split still streams enough KV that its partial stays under ~4% of the bytes it reads.
  const long long partial_bytes = (long long)rows_wg * (d + 2) * 4;
  const long long step_bytes = (long long)kStepTokens * 2 * d * 2;
  long long min_steps = (partial_bytes * 25 + step_bytes - 1) / step_bytes;
  if (min_steps < kWaves) min_steps = kWaves;
  const long long target = (mode == MODE_DENSE) ? 4LL * ncu : ncu;
  long long ns = target / pairs;
  const long long ns_cap = (T + min_steps - 1) / min_steps;
  if (ns > ns_cap) ns = ns_cap;
  if (ns > kMaxSplits) ns = kMaxSplits;
  if (ns < 1) ns = 1;
  // whole rounds of the CUs
  if (pairs * ns > ncu) {
    const long long whole = (pairs * ns) / ncu * ncu / pairs;
    if (whole >= 1) ns = whole;
  }
  p.n_split = (int32_t)ns;
  p.part_bytes = (p.n_split > 1) ? align_up((size_t)pairs * p.n_split * kMaxRowsPerWG * (d + 2) * 4, 256) : 0;
  if (mode == MODE_BLOCK) {
    const size_t ucap = (size_t)n_q * cap;
    p.ublk_bytes = align_up((size_t)B * Hkv * ucap * 4, 256);
    p.umask_bytes = align_up((size_t)B * Hkv * ucap * 8, 256);
    p.ucount_bytes = align_up((size_t)B * Hkv * 4, 256);
  }
  p.total_bytes = p.part_bytes + p.ublk_bytes + p.umask_bytes + p.ucount_bytes;
  if (p.total_bytes == 0) p.total_bytes = 256;
  return p;
}

UnionLayout union_layout(int32_t B, int32_t Hkv, int32_t n_q, int32_t cap) {
  UnionLayout u{};
  const size_t ucap = (size_t)n_q * (cap > 0 ? cap : 0);
  u.ublk_bytes = align_up((size_t)B * Hkv * ucap * 4, 256);
  u.umask_bytes = align_up((size_t)B * Hkv * ucap * 8, 256);
  u.ucount_bytes = align_up((size_t)B * Hkv * 4, 256);
  u.total_bytes = u.ublk_bytes + u.umask_bytes + u.ucount_bytes;
  return u;
}

AttnPlan attn_plan_nsa(int32_t B, int32_t n_q, int32_t Hq, int32_t Hkv, int32_t d, int32_t page_size,
                       int32_t cap, int32_t max_tail_len, int32_t max_cmp, int32_t window, int32_t cus) {
  AttnPlan p{};
  p.D = d;
  const int G = Hq / Hkv;
  p.rows = n_q * G;
  p.n_rc = (p.rows + kMaxRowsPerWG - 1) / kMaxRowsPerWG;
  const int rows_wg = p.rows < kMaxRowsPerWG ? p.rows : kMaxRowsPerWG;
  p.QT = (rows_wg + 15) / 16;
  const long long tail_steps = ((long long)max_tail_len + kStepTokens - 1) / kStepTokens;
  const long long T[3] = {((long long)max_cmp + kStepTokens - 1) / kStepTokens,
                          (long long)n_q * cap * (page_size / kStepTokens) + tail_steps,
                          ((long long)window + kStepTokens - 1) / kStepTokens + tail_steps};
  long long pairs = (long long)B * Hkv * p.n_rc;
  if (pairs < 1) pairs = 1;
  // One round of workgroups over the CUs, shared by the branches so that the branch
  // with the most steps per wave has as few as possible (each split adds kWaves waves).
  // The selection branch streams the rows' block union, whose size only the device
  // knows: between one row's cap blocks (every row shares them) and n_q * cap (none
  // shared).  Its estimate is the geometric mean of those bounds, which keeps the worst
  // relative misestimate smallest.  The call is latency-bound, so no split minimum:
  // every branch gets at least one split, and at most one per kWaves steps of its bound.
  const long long ncu = cus > 0 ? cus : kDefaultCUs;
  long long total = ncu / pairs;
  if (total < 3) total = 3;
  const long long t1_lo = (long long)cap * (page_size / kStepTokens) + tail_steps;
  double est[3] = {(double)T[0], (double)T[1], (double)T[2]};
  if (t1_lo > 0 && T[1] > t1_lo) est[1] = sqrt((double)t1_lo * (double)T[1]);
  long long ns[3], cap_ns[3];
  for (int c = 0; c < 3; ++c) {
    ns[c] = 1;
    cap_ns[c] = (T[c] + kWaves - 1) / kWaves;
    if (cap_ns[c] > kMaxSplits / 3) cap_ns[c] = kMaxSplits / 3;
    if (cap_ns[c] < 1) cap_ns[c] = 1;
  }
  for (long long used = 3; used < total; ++used) {
    int best = -1;
    double worst = 0.0;
    for (int c = 0; c < 3; ++c) {
      const double per = est[c] / (double)ns[c];
      if (ns[c] < cap_ns[c] && per > worst) {
        worst = per;
        best = c;
      }
    }
    if (best < 0) break;
    ++ns[best];
  }
  int n = 0;
  for (int c = 0; c < 3; ++c) {
    p.ns_br[c] = (int32_t)ns[c];
    n += (int32_t)ns[c];
  }
  p.n_split = n;
  p.T_max = (int32_t)(T[0] > T[1] ? (T[0] > T[2] ? T[0] : T[2]) : (T[1] > T[2] ? T[1] : T[2]));
  p.part_bytes = align_up((size_t)pairs * p.n_split * kMaxRowsPerWG * (d + 2) * 4, 256);
  p.total_bytes = p.part_bytes;
  return p;
}

hipError_t union_launch(const AttnArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(block_union_kernel, dim3(a.B * a.Hkv), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t compress_launch(const AttnArgs& a, int32_t d, int32_t B, const int32_t* prefix_len, uint16_t* kc,
                           uint16_t* vc, hipStream_t stream) {
  if (a.max_cmp < 1 || B < 1) return hipSuccess;
  const int per = 256 / (d / 8);                 // compressed rows per workgroup
  const dim3 grid((a.max_cmp + per - 1) / per, a.Hkv, B);
  if (d == 128)
    hipLaunchKernelGGL(compress_kernel<128>, grid, dim3(256), 0, stream, a, prefix_len, kc, vc);
  else
    hipLaunchKernelGGL(compress_kernel<64>, grid, dim3(256), 0, stream, a, prefix_len, kc, vc);
  return hipGetLastError();
}

hipError_t attn_launch(const AttnPlan& p, AttnArgs a, void* workspace, hipStream_t stream) {
  char* ws = static_cast<char*>(workspace);
  a.part = p.part_bytes ? reinterpret_cast<float*>(ws) : nullptr;
  ws += p.part_bytes;
  a.T_max = p.T_max;
  a.n_split = p.n_split;
  a.rows = p.rows;
  a.n_rc = p.n_rc;
  if (a.mode == MODE_NSA) {      // the union plan is the caller's (a.ublk, a.umask, a.ucount)
    a.ns0 = p.ns_br[0];
    a.ns1 = p.ns_br[1];
    a.ns2 = p.ns_br[2];
    return (p.D == 128) ? launch_main<128>(p, a, stream) : launch_main<64>(p, a, stream);
  }
  if (a.mode == MODE_BLOCK) {
    a.ublk = reinterpret_cast<const int32_t*>(ws);
    ws += p.ublk_bytes;
    a.umask = reinterpret_cast<const uint64_t*>(ws);
    ws += p.umask_bytes;
    a.ucount = reinterpret_cast<const int32_t*>(ws);
    a.ucap = a.n_q * a.cap;
    hipLaunchKernelGGL(block_union_kernel, dim3(a.B * a.Hkv), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return (p.D == 128) ? launch_main<128>(p, a, stream) : launch_main<64>(p, a, stream);
}

}  // namespace lcs
