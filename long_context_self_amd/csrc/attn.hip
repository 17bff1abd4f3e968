// Paged GQA attention kernels for gfx950: dense verify with Collect-2-Query logits,
// sparse draft attention over token lists, and block-sparse grouped rows with
// overlap-aware union loads.
//
// What is computed
//  * Vegas page, "The pith" / "Core claim": verification is full attention of the
//    k+1 verifier rows over the whole KV cache; the pre-softmax logits of the first
//    draft row and the bonus row are written out (Figure 6 caption,
//    "Collect-2-Query": two rows only, so the side traffic stays constant in k).
//  * Vegas page, "The pith": drafting attends to the selected prefix entries only.
//  * SSV page, section 4.2 (exact merged-schedule variant) and Figure 5: grouped
//    verifier rows with different block sets load each shared block once; each row
//    keeps its own selection and its own causal boundary (Figure 6 text).
//
// How (gfx950, wave64, MFMA)
//  * One workgroup = 4 waves = one (sequence, KV head, row chunk, split).  Every
//    q-row of the KV group (n_q verifier rows x G query heads) is a row of the MFMA
//    tile, so each K/V byte fetched from HBM serves all G heads and all n_q rows.
//  * A wave consumes 32 cache positions per step.  S^T = K Q^T runs on
//    v_mfma_f32_16x16x32_bf16 with K rows loaded straight from global memory into
//    the A-operand layout (lane = token, 8 contiguous dims); O^T = V^T P^T uses the
//    V rows transposed in registers (8 tokens x 8 dims per lane, v_perm only) and
//    P taken directly from the S^T accumulator layout, so no LDS is touched in the
//    hot loop.  P is split into bf16 hi + lo parts so the PV product keeps ~16
//    mantissa bits of the softmax weights.
//  * Online softmax in base 2 with the running max and sum per q-row kept in the
//    lane that owns the row; the 4 waves' states are merged through LDS in a fixed
//    order, and a split-K combine merges the workgroups' partials in a fixed order,
//    so results are bitwise reproducible.
//  * The kernel is HBM-bound by design (arithmetic intensity ~ n_q*G flop/byte, far
//    below the MFMA ridge); MFMA is used because the VALU alone could not keep up
//    with the 36-row verify tile at full bandwidth.
#include "lcs_internal.h"

#include <math.h>

namespace lcs {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr uint64_t kAll = ~0ull;
constexpr float kLn2 = 0.693147180559945309417f;

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint64_t shfl64(uint64_t v, int src) {
  uint32_t lo = __shfl((uint32_t)v, src);
  uint32_t hi = __shfl((uint32_t)(v >> 32), src);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) {
  return __builtin_bit_cast(float, h << 16);
}

// V rows: DPL dims per lane (8 for d = 128, 4 for d = 64).
template <int DPL> struct VRow;
template <> struct VRow<8> {
  uint32_t w[4];
  __device__ __forceinline__ void load(const uint16_t* p) {
    u32x4 t = *reinterpret_cast<const u32x4*>(p);
    w[0] = t[0]; w[1] = t[1]; w[2] = t[2]; w[3] = t[3];
  }
  __device__ __forceinline__ void zero() { w[0] = w[1] = w[2] = w[3] = 0; }
};
template <> struct VRow<4> {
  uint32_t w[2];
  __device__ __forceinline__ void load(const uint16_t* p) {
    u32x2 t = *reinterpret_cast<const u32x2*>(p);
    w[0] = t[0]; w[1] = t[1];
  }
  __device__ __forceinline__ void zero() { w[0] = w[1] = 0; }
};

// Element e (a bf16) of row r.
template <int DPL>
__device__ __forceinline__ uint32_t velem(const VRow<DPL>& r, int e) {
  return (e & 1) ? (r.w[e >> 1] >> 16) : (r.w[e >> 1] & 0xffffu);
}

template <int D, int KS, int DPL>
struct StepBuf {
  u32x4 k[2][KS];
  VRow<DPL> v[8];
  uint32_t vok;     // bit t set when V token t of this lane is a real cache row
};

struct SeqInfo {
  int L, cnt, tb, tl, U, T;
  const int32_t* list;
  const int32_t* ub;
  const uint64_t* um;
};

// Sequence-level bounds for (b, g); every quantity read from device memory is clamped.
__device__ __forceinline__ SeqInfo seq_info(const AttnArgs& a, int b, int g) {
  SeqInfo si{};
  const int P = 1 << a.lg_page;
  if (a.mode == MODE_DENSE) {
    si.L = min(max(a.prefix_len[b], 0), a.max_prefix_len);
    si.T = (si.L + a.n_q + kStepTokens - 1) / kStepTokens;
  } else {
    si.tb = a.tail_begin[b];
    si.tl = max(a.tail_len[b], 0);
    if (a.mode == MODE_BLOCK) {
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
// Token metadata.  A wave owns a contiguous range of 32-token steps.  For each
// window of kMW steps it builds, one window ahead, the K/V row index and the
// row-visibility mask of every token slot in a per-wave LDS ring, in three
// stages spread over the first three steps of the previous window (positions
// and index-list loads; block-table loads; rows, masks and flags to LDS).  No
// global load therefore sits between a step and the issue of its data loads.
// ---------------------------------------------------------------------------
constexpr int kMW = 4;                      // steps per metadata window
constexpr int kMT = kMW * kStepTokens;      // token slots per window
constexpr int kTokPerLane = kMT / 64;       // slots each lane builds per window

struct WaveMeta {
  int32_t row[2][kMT];
  uint64_t vis[2][kMT];
  uint32_t full[2][kMW];
};

struct MetaStage {
  int pos[kTokPerLane];
  int jt[kTokPerLane];
  int page[kTokPerLane];
  uint64_t v[kTokPerLane];
};

// Stage A: logical position of each slot (index-list loads in list modes).
__device__ __forceinline__ void meta_stage_a(const AttnArgs& a, const SeqInfo& si, int wbase, int w1,
                                             int lane, MetaStage& ms) {
  const int P = 1 << a.lg_page;
#pragma unroll
  for (int r = 0; r < kTokPerLane; ++r) {
    const int tok = lane + 64 * r;
    const int step = wbase + tok / kStepTokens;
    const int t = tok & (kStepTokens - 1);
    int pos = -1, jt = -1;
    uint64_t v = 0;
    if (step < w1) {
      if (a.mode == MODE_DENSE) {
        const int u = step * kStepTokens + t;
        if (u < si.L) {
          pos = u;
          v = kAll;
        } else if (u < si.L + a.n_q) {
          pos = u;
          jt = u - si.L;
        }
      } else if (a.mode == MODE_BLOCK) {
        const int spb = P / kStepTokens;
        const int blk_steps = si.U * spb;
        if (step < blk_steps) {
          const int e = step / spb;
          const int blk = si.ub[e];
          const int p = blk * P + (step - e * spb) * kStepTokens + t;
          if (blk >= 0 && blk < a.max_pages && p < si.tb) {
            pos = p;
            v = si.um[e];
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
        // the index load is issued for every slot (clamped), keeping wait counts static
        const int32_t* src = (si.cnt > 0) ? si.list + min(max(u, 0), si.cnt - 1) : a.bt;
        const int lp = *src;
        if (u < si.cnt) {
          pos = lp;
          v = kAll;
        } else if (u - si.cnt < si.tl) {
          jt = u - si.cnt;
          pos = si.tb + jt;
        }
      }
    }
    ms.pos[r] = pos;
    ms.jt[r] = jt;
    ms.v[r] = v;
  }
}

// Stage B: physical page of each slot (block-table loads).
__device__ __forceinline__ void meta_stage_b(const AttnArgs& a, int b, MetaStage& ms) {
#pragma unroll
  for (int r = 0; r < kTokPerLane; ++r) {
    const int pos = ms.pos[r];
    const int pi = pos >> a.lg_page;
    const bool ok = pos >= 0 && pi < a.max_pages;
    // issued for every slot (clamped in range), keeping wait counts static
    const int page = a.bt[(size_t)b * a.max_pages + (ok ? pi : 0)];
    ms.page[r] = ok ? page : -1;
  }
}

// Stage C: row index, visibility mask and per-step "everything visible" flag to LDS.
__device__ __forceinline__ void meta_stage_c(const AttnArgs& a, int g, uint64_t colmask, int lane,
                                             const MetaStage& ms, WaveMeta& wm, int buf) {
  const int P = 1 << a.lg_page;
#pragma unroll
  for (int r = 0; r < kTokPerLane; ++r) {
    const int tok = lane + 64 * r;
    const int jt = ms.jt[r];
    const uint64_t cm = shfl64(colmask, jt & 63);     // every lane takes part in the shuffle
    uint64_t v = ms.v[r];
    if (jt >= 0) v = (jt < 64 || a.rowmask == nullptr) ? cm : 0;
    int row = -1;
    const int page = ms.page[r];
    if ((unsigned)page < (unsigned)a.num_pages) row = ((page * a.Hkv + g) << a.lg_page) | (ms.pos[r] & (P - 1));
    if (row < 0) v = 0;
    wm.row[buf][tok] = row;
    wm.vis[buf][tok] = v;
    const uint64_t ok = __ballot(row >= 0 && v == kAll);
    if (lane == 0) {
      wm.full[buf][2 * r] = (uint32_t)ok == 0xffffffffu;
      wm.full[buf][2 * r + 1] = (uint32_t)(ok >> 32) == 0xffffffffu;
    }
  }
}

// Issue the K and V loads of local step ls of window buffer buf.
template <int D, int KS, int DPL>
__device__ __forceinline__ void step_load(const AttnArgs& a, const WaveMeta& wm, int buf, int ls, int x,
                                          int j, StepBuf<D, KS, DPL>& sb) {
  const int32_t* rows = wm.row[buf] + ls * kStepTokens;
  const int rk0 = rows[x];
  const int rk1 = rows[16 + x];
  const uint16_t* k0 = a.k + (size_t)max(rk0, 0) * D + 8 * j;
  const uint16_t* k1 = a.k + (size_t)max(rk1, 0) * D + 8 * j;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    sb.k[0][ks] = *reinterpret_cast<const u32x4*>(k0 + 32 * ks);
    sb.k[1][ks] = *reinterpret_cast<const u32x4*>(k1 + 32 * ks);
  }
  const int4 rv0 = *reinterpret_cast<const int4*>(rows + 4 * j);
  const int4 rv1 = *reinterpret_cast<const int4*>(rows + 16 + 4 * j);
  const int rv[8] = {rv0.x, rv0.y, rv0.z, rv0.w, rv1.x, rv1.y, rv1.z, rv1.w};
  // every load is issued (invalid slots read row 0) so the wait counts stay static;
  // invalid rows are zeroed at use, since a masked weight times a NaN would poison O
  uint32_t vok = 0;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    sb.v[t].load(a.v + (size_t)max(rv[t], 0) * D + DPL * x);
    vok |= (rv[t] >= 0 ? 1u : 0u) << t;
  }
  sb.vok = vok;
}

template <int D, int QT>
__global__ void __launch_bounds__(256) attn_kernel(AttnArgs a) {
  constexpr int DPL = D / 16;   // dims per lane per token in the V^T operand
  constexpr int KS = D / 32;    // k-steps of the QK^T product
  constexpr int QLD = D + 8;    // LDS row stride of Q in bf16 (pads bank conflicts away)
  constexpr int kPer = 4 * DPL + 2;                       // merge floats per lane per q-tile
  constexpr size_t kQBytes = (size_t)QT * 16 * QLD * 2;
  constexpr size_t kMetaBytes = sizeof(WaveMeta) * kWaves;
  constexpr size_t kMergeBytes = (size_t)(kWaves - 1) * QT * kPer * 64 * 4;
  constexpr size_t kLoopBytes = kQBytes + kMetaBytes;
  constexpr size_t kSmem = kLoopBytes > kMergeBytes ? kLoopBytes : kMergeBytes;
  __shared__ __attribute__((aligned(16))) unsigned char smem_raw[kSmem];
  uint16_t* s_q = reinterpret_cast<uint16_t*>(smem_raw);
  WaveMeta* s_meta = reinterpret_cast<WaveMeta*>(smem_raw + kQBytes);
  float* s_merge = reinterpret_cast<float*>(smem_raw);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int x = lane & 15;
  const int j = lane >> 4;
  const int s = blockIdx.x;
  const int g = blockIdx.y % a.Hkv;
  const int rc = blockIdx.y / a.Hkv;
  const int b = blockIdx.z;
  const int r0 = rc * kMaxRowsPerWG;
  const int nrows = min(kMaxRowsPerWG, a.rows - r0);
  WaveMeta& wm = s_meta[wave];

  // Q rows of this workgroup -> LDS (rows past nrows are zero)
  for (int e = tid; e < QT * 16 * (D / 8); e += 256) {
    const int r = e / (D / 8);
    const int c = e - r * (D / 8);
    u32x4 v = u32x4{0, 0, 0, 0};
    if (r < nrows) {
      const int rr = r0 + r;
      const int i = rr / a.G;
      const int h = g * a.G + (rr - i * a.G);
      v = *reinterpret_cast<const u32x4*>(a.q + ((size_t)(b * a.n_q + i) * a.Hq + h) * D + 8 * c);
    }
    *reinterpret_cast<u32x4*>(s_q + r * QLD + 8 * c) = v;
  }

  const SeqInfo si = seq_info(a, b, g);
  const int st0 = s * a.sps;
  const int st1 = (s == a.n_split - 1) ? si.T : min(si.T, st0 + a.sps);
  // contiguous per-wave step ranges
  const int nst = max(st1 - st0, 0);
  const int qw = (nst + kWaves - 1) / kWaves;
  const int w0 = st0 + wave * qw;
  const int w1 = min(st1, w0 + qw);

  // Column mask of verifier/tail slot `lane`: bit i = row i sees that slot.
  uint64_t colmask;
  if (a.rowmask != nullptr) {
    colmask = 0;
    const uint64_t* rm = a.rowmask + (size_t)b * a.n_q;
    for (int i = 0; i < a.n_q; ++i) colmask |= ((rm[i] >> lane) & 1ull) << i;
  } else {
    colmask = (a.mode == MODE_DENSE) ? (kAll << lane) : kAll;
  }

  // verifier row index of this lane's q-row in each tile (64 = padding row)
  int rowi[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int r = 16 * qt + x;
    rowi[qt] = (r < nrows) ? (r0 + r) / a.G : 64;
  }
  const bool collect = a.mode == MODE_DENSE && a.logits != nullptr;

  float m[QT], l[QT];
  f32x4 O[QT][DPL];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    m[qt] = -INFINITY;
    l[qt] = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) O[qt][e] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  __syncthreads();   // Q in LDS

  if (w0 < w1) {
    MetaStage ms;
    meta_stage_a(a, si, w0, w1, lane, ms);
    meta_stage_b(a, b, ms);
    meta_stage_c(a, g, colmask, lane, ms, wm, 0);
    StepBuf<D, KS, DPL> cur;
    step_load<D, KS, DPL>(a, wm, 0, 0, x, j, cur);
    for (int wb = w0, k = 0; wb < w1; wb += kMW, ++k) {
      const int buf = k & 1;
      const bool next_win = wb + kMW < w1;
      const int nloc = min(kMW, w1 - wb);
      for (int ls = 0; ls < nloc; ++ls) {
        const int step = wb + ls;
        if (next_win) {
          if (ls == 0) meta_stage_a(a, si, wb + kMW, w1, lane, ms);
          if (ls == 1) meta_stage_b(a, b, ms);
          if (ls == 2) meta_stage_c(a, g, colmask, lane, ms, wm, buf ^ 1);
        }
        // next step's loads go out before this step is consumed (the last step re-reads itself)
        StepBuf<D, KS, DPL> nxt;
        {
          int nb = buf, nls = ls + 1;
          if (nls == kMW) { nb = buf ^ 1; nls = 0; }
          if (step + 1 >= w1) { nb = buf; nls = ls; }
          step_load<D, KS, DPL>(a, wm, nb, nls, x, j, nxt);
        }

        // ---- S^T = K Q^T for two 16-token tiles (Q^T operand from LDS)
        f32x4 S[2][QT];
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          S[0][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
          S[1][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const u32x4 qop = *reinterpret_cast<const u32x4*>(s_q + (16 * qt + x) * QLD + 32 * ks + 8 * j);
            S[0][qt] = mfma16(cur.k[0][ks], qop, S[0][qt]);
            S[1][qt] = mfma16(cur.k[1][ks], qop, S[1][qt]);
          }
        }

        // ---- visibility of the 8 tokens this lane holds (tokens 16tt + 4j + i)
        const bool full = wm.full[buf][ls] != 0;
        uint64_t vt[2][4];
        if (!full) {
          const uint64_t* vr = wm.vis[buf] + ls * kStepTokens;
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) vt[tt][i] = vr[16 * tt + 4 * j + i];
        }

        // ---- online softmax per q-tile; P as bf16 hi + lo B-operands
        u32x4 phi[QT], plo[QT];
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          float t8[8];
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float sv = S[tt][qt][i] * a.scale_log2;
              if (!full && ((vt[tt][i] >> rowi[qt]) & 1ull) == 0) sv = -INFINITY;
              t8[4 * tt + i] = sv;
            }
          // Collect-2-Query: scaled logits of the two collected rows, prefix columns only
          if (collect && (rowi[qt] == a.c0 || rowi[qt] == a.c1)) {
            const int rr = r0 + 16 * qt + x;
            const int h = g * a.G + (rr - rowi[qt] * a.G);
            float* base = a.logits + (size_t)(b * a.Hq + h) * 2 * a.logits_ld;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
              if (rowi[qt] != (c == 0 ? a.c0 : a.c1)) continue;
              float* dst = base + c * a.logits_ld;
#pragma unroll
              for (int tt = 0; tt < 2; ++tt) {
                const int p0 = step * kStepTokens + 16 * tt + 4 * j;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                  if (p0 + i < si.L) dst[p0 + i] = S[tt][qt][i] * a.scale;
              }
            }
          }
          float rmax = t8[0];
#pragma unroll
          for (int u = 1; u < 8; ++u) rmax = fmaxf(rmax, t8[u]);
          rmax = fmaxf(rmax, __shfl_xor(rmax, 16));
          rmax = fmaxf(rmax, __shfl_xor(rmax, 32));
          const float mnew = fmaxf(m[qt], rmax);
          const float msafe = (mnew == -INFINITY) ? 0.f : mnew;
          const float alpha = __builtin_amdgcn_exp2f(m[qt] - msafe);
          m[qt] = mnew;
          float psum = 0.f;
#pragma unroll
          for (int u = 0; u < 8; u += 2) {
            const float p0 = __builtin_amdgcn_exp2f(t8[u] - msafe);
            const float p1 = __builtin_amdgcn_exp2f(t8[u + 1] - msafe);
            psum += p0 + p1;
            const uint32_t h0 = bf16_rne(p0), h1 = bf16_rne(p1);
            const uint32_t l0 = bf16_rne(p0 - bf16_to_f32(h0));
            const uint32_t l1 = bf16_rne(p1 - bf16_to_f32(h1));
            phi[qt][u >> 1] = h0 | (h1 << 16);
            plo[qt][u >> 1] = l0 | (l1 << 16);
          }
          l[qt] = l[qt] * alpha + psum;
          if (__any(alpha != 1.f)) {
#pragma unroll
            for (int e = 0; e < DPL; ++e) O[qt][e] *= alpha;
          }
        }

        // ---- O^T += V^T P^T, one transposed V tile at a time
#pragma unroll
        for (int e = 0; e < DPL; ++e) {
          u32x4 vte;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const uint32_t lo = (cur.vok >> (2 * w)) & 1u ? velem<DPL>(cur.v[2 * w], e) : 0u;
            const uint32_t hi = (cur.vok >> (2 * w + 1)) & 1u ? velem<DPL>(cur.v[2 * w + 1], e) : 0u;
            vte[w] = lo | (hi << 16);
          }
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) {
            O[qt][e] = mfma16(vte, phi[qt], O[qt][e]);
            O[qt][e] = mfma16(vte, plo[qt], O[qt][e]);
          }
        }
        cur = nxt;
      }
    }
  }

  // full row sums (fixed order)
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    l[qt] += __shfl_xor(l[qt], 16);
    l[qt] += __shfl_xor(l[qt], 32);
  }

  // ---- merge the 4 waves' states through LDS in wave order 0,1,2,3
  __syncthreads();   // every wave is done with Q and its metadata ring
  if (wave > 0) {
    float* w = s_merge + (size_t)(wave - 1) * QT * kPer * 64;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
      for (int e = 0; e < DPL; ++e)
#pragma unroll
        for (int i = 0; i < 4; ++i) w[(qt * kPer + e * 4 + i) * 64 + lane] = O[qt][e][i];
      w[(qt * kPer + 4 * DPL) * 64 + lane] = m[qt];
      w[(qt * kPer + 4 * DPL + 1) * 64 + lane] = l[qt];
    }
  }
  __syncthreads();
  if (wave != 0) return;
  for (int ow = 1; ow < kWaves; ++ow) {
    const float* w = s_merge + (size_t)(ow - 1) * QT * kPer * 64;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float mb = w[(qt * kPer + 4 * DPL) * 64 + lane];
      const float lb = w[(qt * kPer + 4 * DPL + 1) * 64 + lane];
      const float M = fmaxf(m[qt], mb);
      const float Ms = (M == -INFINITY) ? 0.f : M;
      const float wa = __builtin_amdgcn_exp2f(m[qt] - Ms);
      const float wb = __builtin_amdgcn_exp2f(mb - Ms);
      m[qt] = M;
      l[qt] = wa * l[qt] + wb * lb;
#pragma unroll
      for (int e = 0; e < DPL; ++e)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          O[qt][e][i] = wa * O[qt][e][i] + wb * w[(qt * kPer + e * 4 + i) * 64 + lane];
    }
  }

  // ---- write: final output when there is a single split, else a partial
  const size_t pstride = (size_t)kMaxRowsPerWG * (D + 2);
  const size_t pidx = ((size_t)(b * a.Hkv + g) * a.n_rc + rc) * a.n_split + s;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int r = 16 * qt + x;
    if (r >= nrows) continue;
    const int d0 = 4 * DPL * j;
    if (a.n_split == 1) {
      const int rr = r0 + r;
      const int i = rr / a.G;
      const int h = g * a.G + (rr - i * a.G);
      const float inv = (l[qt] > 0.f) ? 1.f / l[qt] : 0.f;
      float* op = a.out + ((size_t)(b * a.n_q + i) * a.Hq + h) * D + d0;
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
#pragma unroll
        for (int e4 = 0; e4 < DPL; e4 += 4) {
          f32x4 v4 = f32x4{O[qt][e4][i4], O[qt][e4 + 1][i4], O[qt][e4 + 2][i4], O[qt][e4 + 3][i4]};
          *reinterpret_cast<f32x4*>(op + DPL * i4 + e4) = v4 * inv;
        }
      if (j == 0 && a.lse != nullptr)
        a.lse[(size_t)(b * a.n_q + i) * a.Hq + h] =
            (l[qt] > 0.f) ? (m[qt] + __log2f(l[qt])) * kLn2 : -INFINITY;
    } else {
      float* pp = a.part + pidx * pstride;
      float* op = pp + (size_t)r * D + d0;
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
#pragma unroll
        for (int e4 = 0; e4 < DPL; e4 += 4)
          *reinterpret_cast<f32x4*>(op + DPL * i4 + e4) =
              f32x4{O[qt][e4][i4], O[qt][e4 + 1][i4], O[qt][e4 + 2][i4], O[qt][e4 + 3][i4]};
      if (j == 0) {
        pp[(size_t)kMaxRowsPerWG * D + r] = m[qt];
        pp[(size_t)kMaxRowsPerWG * D + kMaxRowsPerWG + r] = l[qt];
      }
    }
  }
}

// Merge split-K partials in split order.  One wave per q-row: lane s first loads the
// (m, l) of split s, so the per-split loads are issued together rather than one
// after another; then every lane accumulates its columns over the splits.
constexpr int kCombineRows = 4;

template <int D>
__global__ void __launch_bounds__(256) combine_kernel(AttnArgs a) {
  const int pid = blockIdx.x;                   // (b*Hkv + g)*n_rc + rc
  const int rc = pid % a.n_rc;
  const int bg = pid / a.n_rc;
  const int g = bg % a.Hkv;
  const int b = bg / a.Hkv;
  const int r0 = rc * kMaxRowsPerWG;
  const int nrows = min(kMaxRowsPerWG, a.rows - r0);
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.y * kCombineRows + (threadIdx.x >> 6);
  if (r >= nrows) return;
  const size_t pstride = (size_t)kMaxRowsPerWG * (D + 2);
  const float* base = a.part + (size_t)pid * a.n_split * pstride;
  const float* mcol = base + (size_t)kMaxRowsPerWG * D + r;
  // splits are at most kMaxSplits = 128: two per lane
  float mv[2], lv[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int sp = lane + 64 * u;
    mv[u] = (sp < a.n_split) ? mcol[sp * pstride] : -INFINITY;
    lv[u] = (sp < a.n_split) ? mcol[sp * pstride + kMaxRowsPerWG] : 0.f;
  }
  float M = fmaxf(mv[0], mv[1]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  const float Ms = (M == -INFINITY) ? 0.f : M;
  float wv[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) wv[u] = __builtin_amdgcn_exp2f(mv[u] - Ms);
  // L = sum over splits in split order: gather the weighted l's to lane 0's order via LDS
  __shared__ float s_w[kCombineRows][kMaxSplits];
  __shared__ float s_l[kCombineRows][kMaxSplits];
  const int wr = threadIdx.x >> 6;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    s_w[wr][lane + 64 * u] = wv[u];
    s_l[wr][lane + 64 * u] = wv[u] * lv[u];
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  float Ls = 0.f;
  for (int sp = 0; sp < a.n_split; ++sp) Ls += s_l[wr][sp];
  constexpr int CPL = D / 64;                   // columns per lane (2 or 1)
  float acc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
  const float* ocol = base + (size_t)r * D + CPL * lane;
  int sp = 0;
  for (; sp + 4 <= a.n_split; sp += 4) {
    float ov[4][CPL];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int c = 0; c < CPL; ++c) ov[u][c] = ocol[(sp + u) * pstride + c];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[c] += s_w[wr][sp + u] * ov[u][c];
  }
  for (; sp < a.n_split; ++sp)
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] += s_w[wr][sp] * ocol[sp * pstride + c];
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

// Union of the n_q rows' block lists of one (b, g), ascending, with per-block row masks
// (SSV page, section 4.2: shared blocks are scheduled once for the whole group).
constexpr int kPlanChunk = 4096;

__global__ void __launch_bounds__(256) block_union_kernel(AttnArgs a) {
  const int bg = blockIdx.x;
  const int g = bg % a.Hkv;
  const int b = bg / a.Hkv;
  const int tid = threadIdx.x;
  __shared__ uint32_t mlo[kPlanChunk];
  __shared__ uint32_t mhi[kPlanChunk];
  __shared__ uint32_t tsum[256];
  int32_t* ub = const_cast<int32_t*>(a.ublk) + (size_t)bg * a.ucap;
  uint64_t* um = const_cast<uint64_t*>(a.umask) + (size_t)bg * a.ucap;
  int total = 0;
  for (int base = 0; base < a.max_pages; base += kPlanChunk) {
    for (int e = tid; e < kPlanChunk; e += 256) mlo[e] = mhi[e] = 0;
    __syncthreads();
    for (int i = 0; i < a.n_q && a.cap > 0; ++i) {
      const size_t o = (size_t)(b * a.n_q + i) * a.Hkv + g;
      const int cnt = min(max(a.counts[o], 0), a.cap);
      const int32_t* lst = a.indices + o * a.cap;
      for (int e = tid; e < cnt; e += 256) {
        const int blk = lst[e];
        if (blk >= base && blk < base + kPlanChunk && blk < a.max_pages) {
          if (i < 32) atomicOr(&mlo[blk - base], 1u << i);
          else atomicOr(&mhi[blk - base], 1u << (i - 32));
        }
      }
    }
    __syncthreads();
    // ascending compaction: thread t owns ids [16t, 16t + 16)
    uint32_t c = 0;
    for (int e = 0; e < 16; ++e) c += (mlo[16 * tid + e] | mhi[16 * tid + e]) != 0;
    tsum[tid] = c;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const uint32_t v = (tid >= off) ? tsum[tid - off] : 0;
      __syncthreads();
      tsum[tid] += v;
      __syncthreads();
    }
    uint32_t w = total + tsum[tid] - c;
    for (int e = 0; e < 16; ++e) {
      const int id = 16 * tid + e;
      const uint64_t msk = ((uint64_t)mhi[id] << 32) | mlo[id];
      if (msk != 0 && (int)w < a.ucap) {
        ub[w] = base + id;
        um[w] = msk;
        ++w;
      }
    }
    total += tsum[255];
    __syncthreads();
  }
  if (tid == 0) const_cast<int32_t*>(a.ucount)[bg] = min(total, a.ucap);
}

template <int D>
hipError_t launch_main(const AttnPlan& p, const AttnArgs& a, hipStream_t stream) {
  dim3 grid(p.n_split, a.Hkv * p.n_rc, a.B);
  switch (p.QT) {
    case 1: hipLaunchKernelGGL((attn_kernel<D, 1>), grid, dim3(256), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((attn_kernel<D, 2>), grid, dim3(256), 0, stream, a); break;
    case 3: hipLaunchKernelGGL((attn_kernel<D, 3>), grid, dim3(256), 0, stream, a); break;
    default: hipLaunchKernelGGL((attn_kernel<D, 4>), grid, dim3(256), 0, stream, a); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_split == 1) return e;
  const int rows_wg = p.rows < kMaxRowsPerWG ? p.rows : kMaxRowsPerWG;
  hipLaunchKernelGGL((combine_kernel<D>), dim3(a.B * a.Hkv * p.n_rc, (rows_wg + kCombineRows - 1) / kCombineRows),
                     dim3(64 * kCombineRows), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

AttnPlan attn_plan(int32_t mode, int32_t B, int32_t n_q, int32_t Hq, int32_t Hkv, int32_t d,
                   int32_t page_size, int32_t max_prefix_len, int32_t cap, int32_t max_tail_len) {
  AttnPlan p{};
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
  // a split streams enough KV that its partial stays under ~4% of the bytes it reads
  const long long partial_bytes = (long long)rows_wg * (d + 2) * 4;
  const long long step_bytes = (long long)kStepTokens * 2 * d * 2;
  long long min_steps = (partial_bytes * 25 + step_bytes - 1) / step_bytes;
  if (min_steps < kWaves) min_steps = kWaves;
  long long ns = (kTargetWGs + pairs - 1) / pairs;
  const long long ns_cap = (T + min_steps - 1) / min_steps;
  if (ns > ns_cap) ns = ns_cap;
  if (ns > kMaxSplits) ns = kMaxSplits;
  if (ns < 1) ns = 1;
  // one workgroup per CU at a time: fill whole rounds of the 256 CUs
  if (pairs * ns > kNumCUs) {
    const long long whole = (pairs * ns) / kNumCUs * kNumCUs / pairs;
    if (whole >= 1) ns = whole;
  }
  p.n_split = (int32_t)ns;
  p.sps = (int32_t)((T + ns - 1) / ns);
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

hipError_t attn_launch(const AttnPlan& p, AttnArgs a, void* workspace, hipStream_t stream) {
  char* ws = static_cast<char*>(workspace);
  a.part = p.part_bytes ? reinterpret_cast<float*>(ws) : nullptr;
  ws += p.part_bytes;
  a.n_split = p.n_split;
  a.sps = p.sps;
  a.rows = p.rows;
  a.n_rc = p.n_rc;
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
