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

// Token slot metadata for one step: each lane computes slot (lane & 31).
// row = K/V row index ((page*Hkv + g)*P + slot) or -1; vis = bit i set when
// verifier row i may attend to the token.
__device__ __forceinline__ void step_meta(const AttnArgs& a, const SeqInfo& si, int b, int g,
                                          int step, uint64_t colmask, int lane, int& row,
                                          uint64_t& vis) {
  const int t = lane & 31;
  const int lgP = a.lg_page;
  const int P = 1 << lgP;
  int pos = -1;
  int jt = -1;          // tail slot index, or -1
  uint64_t v = 0;
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
      const int sub = step - e * spb;
      const int blk = si.ub[e];
      const uint64_t m = si.um[e];
      const int p = blk * P + sub * kStepTokens + t;
      if (blk >= 0 && blk < a.max_pages && p < si.tb) {
        pos = p;
        v = m;
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
      pos = si.list[u];
      v = kAll;
    } else if (u - si.cnt < si.tl) {
      jt = u - si.cnt;
      pos = si.tb + jt;
    }
  }
  // tail visibility comes from the column mask held by lane jt (all lanes shuffle)
  const uint64_t cm = shfl64(colmask, jt & 63);
  if (jt >= 0) v = (jt < 64 || a.rowmask == nullptr) ? cm : 0;
  row = -1;
  if (pos >= 0 && (pos >> lgP) < a.max_pages) {
    const int page = a.bt[(size_t)b * a.max_pages + (pos >> lgP)];
    if ((unsigned)page < (unsigned)a.num_pages) row = ((page * a.Hkv + g) << lgP) | (pos & (P - 1));
  }
  if (row < 0) v = 0;
  vis = v;
}

template <int D, int KS, int DPL>
__device__ __forceinline__ void step_load(const AttnArgs& a, int row, int x, int j,
                                          StepBuf<D, KS, DPL>& buf) {
  const int rk0 = __shfl(row, x);
  const int rk1 = __shfl(row, 16 + x);
  const uint16_t* k0 = a.k + (size_t)max(rk0, 0) * D + 8 * j;
  const uint16_t* k1 = a.k + (size_t)max(rk1, 0) * D + 8 * j;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    buf.k[0][ks] = *reinterpret_cast<const u32x4*>(k0 + 32 * ks);
    buf.k[1][ks] = *reinterpret_cast<const u32x4*>(k1 + 32 * ks);
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int tok = (t < 4) ? (4 * j + t) : (12 + 4 * j + t);
    const int rv = __shfl(row, tok);
    if (rv >= 0)
      buf.v[t].load(a.v + (size_t)rv * D + DPL * x);
    else
      buf.v[t].zero();
  }
}

template <int D, int QT>
__global__ void __launch_bounds__(256) attn_kernel(AttnArgs a) {
  constexpr int DPL = D / 16;   // dims per lane per token in the V^T operand
  constexpr int KS = D / 32;    // k-steps of the QK^T product
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

  const SeqInfo si = seq_info(a, b, g);
  const int st0 = s * a.sps;
  const int st1 = (s == a.n_split - 1) ? si.T : min(si.T, st0 + a.sps);

  // Column mask of verifier/tail slot `lane`: bit i = row i sees that slot.
  uint64_t colmask;
  if (a.rowmask != nullptr) {
    colmask = 0;
    const uint64_t* rm = a.rowmask + (size_t)b * a.n_q;
    for (int i = 0; i < a.n_q; ++i) colmask |= ((rm[i] >> lane) & 1ull) << i;
  } else {
    colmask = (a.mode == MODE_DENSE) ? (kAll << lane) : kAll;
  }

  uint64_t rowbit[QT];
  u32x4 qop[QT][KS];
  float* lgp[QT][2];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int r = 16 * qt + x;
    rowbit[qt] = 0;
    lgp[qt][0] = lgp[qt][1] = nullptr;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qop[qt][ks] = u32x4{0, 0, 0, 0};
    if (r < nrows) {
      const int rr = r0 + r;
      const int i = rr / a.G;
      const int h = g * a.G + (rr - i * a.G);
      rowbit[qt] = 1ull << i;
      const uint16_t* qp = a.q + ((size_t)(b * a.n_q + i) * a.Hq + h) * D + 8 * j;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qop[qt][ks] = *reinterpret_cast<const u32x4*>(qp + 32 * ks);
      if (a.mode == MODE_DENSE && a.logits != nullptr) {
        float* base = a.logits + (size_t)(b * a.Hq + h) * 2 * a.logits_ld;
        if (i == a.c0) lgp[qt][0] = base;
        if (i == a.c1) lgp[qt][1] = base + a.logits_ld;
      }
    }
  }

  float m[QT], l[QT];
  f32x4 O[QT][DPL];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    m[qt] = -INFINITY;
    l[qt] = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) O[qt][e] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  int step = st0 + wave;
  StepBuf<D, KS, DPL> cur;
  int row_c = -1;
  uint64_t vis_c = 0;
  if (step < st1) {
    step_meta(a, si, b, g, step, colmask, lane, row_c, vis_c);
    step_load<D, KS, DPL>(a, row_c, x, j, cur);
  }
  for (; step < st1; step += kWaves) {
    // issue the next step's loads before consuming this one
    const int nstep = step + kWaves;
    StepBuf<D, KS, DPL> nxt;
    int row_n = -1;
    uint64_t vis_n = 0;
    if (nstep < st1) {
      step_meta(a, si, b, g, nstep, colmask, lane, row_n, vis_n);
      step_load<D, KS, DPL>(a, row_n, x, j, nxt);
    }

    // ---- S^T = K Q^T for two 16-token tiles
    f32x4 S[2][QT];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc = mfma16(cur.k[tt][ks], qop[qt][ks], acc);
        S[tt][qt] = acc;
      }

    // ---- visibility of the 8 tokens this lane holds (tokens 16tt + 4j + i)
    const bool full = __all(row_c >= 0 && vis_c == kAll);
    uint64_t vt[2][4];
    if (!full) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) vt[tt][i] = shfl64(vis_c, 16 * tt + 4 * j + i);
    }

    // ---- V^T operands: transpose 8 tokens x DPL dims per lane
    u32x4 VT[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e)
#pragma unroll
      for (int w = 0; w < 4; ++w)
        VT[e][w] = velem<DPL>(cur.v[2 * w], e) | (velem<DPL>(cur.v[2 * w + 1], e) << 16);

#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float t8[8];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float sv = S[tt][qt][i] * a.scale_log2;
          if (!full && (vt[tt][i] & rowbit[qt]) == 0) sv = -INFINITY;
          t8[4 * tt + i] = sv;
        }
      // Collect-2-Query: scaled logits of the two collected rows, prefix columns only
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        float* dst = lgp[qt][c];
        if (dst != nullptr) {
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
      u32x4 phi, plo;
#pragma unroll
      for (int u = 0; u < 8; u += 2) {
        const float p0 = __builtin_amdgcn_exp2f(t8[u] - msafe);
        const float p1 = __builtin_amdgcn_exp2f(t8[u + 1] - msafe);
        psum += p0 + p1;
        const uint32_t h0 = bf16_rne(p0), h1 = bf16_rne(p1);
        const uint32_t l0 = bf16_rne(p0 - bf16_to_f32(h0));
        const uint32_t l1 = bf16_rne(p1 - bf16_to_f32(h1));
        phi[u >> 1] = h0 | (h1 << 16);
        plo[u >> 1] = l0 | (l1 << 16);
      }
      l[qt] = l[qt] * alpha + psum;
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        O[qt][e] *= alpha;
        O[qt][e] = mfma16(VT[e], phi, O[qt][e]);
        O[qt][e] = mfma16(VT[e], plo, O[qt][e]);
      }
    }

    cur = nxt;
    row_c = row_n;
    vis_c = vis_n;
  }

  // full row sums (fixed order)
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    l[qt] += __shfl_xor(l[qt], 16);
    l[qt] += __shfl_xor(l[qt], 32);
  }

  // ---- merge the 4 waves' states through LDS in wave order 0,1,2,3
  constexpr int kPer = 4 * DPL + 2;   // floats per lane per q-tile
  __shared__ float smem[(kWaves - 1) * QT * kPer * 64];
  if (wave > 0) {
    float* w = smem + (size_t)(wave - 1) * QT * kPer * 64;
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
    const float* w = smem + (size_t)(ow - 1) * QT * kPer * 64;
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

// Merge split-K partials of one (b, g, row chunk) in split order.
template <int D>
__global__ void __launch_bounds__(256) combine_kernel(AttnArgs a) {
  const int pid = blockIdx.x;
  const int rc = pid % a.n_rc;
  const int bg = pid / a.n_rc;
  const int g = bg % a.Hkv;
  const int b = bg / a.Hkv;
  const int r0 = rc * kMaxRowsPerWG;
  const int nrows = min(kMaxRowsPerWG, a.rows - r0);
  const size_t pstride = (size_t)kMaxRowsPerWG * (D + 2);
  const float* base = a.part + (size_t)pid * a.n_split * pstride;
  __shared__ float wsh[kMaxSplits][kMaxRowsPerWG];
  __shared__ float inv[kMaxRowsPerWG];
  const int tid = threadIdx.x;
  if (tid < nrows) {
    float M = -INFINITY;
    for (int s = 0; s < a.n_split; ++s) M = fmaxf(M, base[s * pstride + kMaxRowsPerWG * D + tid]);
    const float Ms = (M == -INFINITY) ? 0.f : M;
    float Ls = 0.f;
    for (int s = 0; s < a.n_split; ++s) {
      const float ms = base[s * pstride + kMaxRowsPerWG * D + tid];
      const float ws = __builtin_amdgcn_exp2f(ms - Ms);
      wsh[s][tid] = ws;
      Ls += ws * base[s * pstride + kMaxRowsPerWG * D + kMaxRowsPerWG + tid];
    }
    inv[tid] = (Ls > 0.f) ? 1.f / Ls : 0.f;
    if (a.lse != nullptr) {
      const int rr = r0 + tid;
      const int i = rr / a.G;
      const int h = g * a.G + (rr - i * a.G);
      a.lse[(size_t)(b * a.n_q + i) * a.Hq + h] = (Ls > 0.f) ? (M + __log2f(Ls)) * kLn2 : -INFINITY;
    }
  }
  __syncthreads();
  constexpr int C4 = D / 4;
  for (int item = tid; item < nrows * C4; item += blockDim.x) {
    const int r = item / C4;
    const int c = item - r * C4;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < a.n_split; ++s)
      acc += wsh[s][r] * *reinterpret_cast<const f32x4*>(base + s * pstride + (size_t)r * D + 4 * c);
    const int rr = r0 + r;
    const int i = rr / a.G;
    const int h = g * a.G + (rr - i * a.G);
    *reinterpret_cast<f32x4*>(a.out + ((size_t)(b * a.n_q + i) * a.Hq + h) * D + 4 * c) = acc * inv[r];
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
  hipLaunchKernelGGL((combine_kernel<D>), dim3(a.B * a.Hkv * p.n_rc), dim3(256), 0, stream, a);
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
