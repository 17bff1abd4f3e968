// Verification-guided top-k selection for gfx950.
//
// What is computed
//  * Vegas page, "Core claim" / "What carries the argument": the logits of the
//    first draft row and the bonus row are combined across the query heads and
//    the k prefix positions with the largest combined score are kept.
//  * Sparse Glimpse page, "Core claim": sink + recent + top-ranked history, one
//    set per head (here per KV head, scored over the heads of its group).
//  * SSV page, NSA block selection: a block scores the max of its positions, or
//    (the alternative aggregation) their log-sum-exp, m + log(sum exp(sigma_p - m)),
//    computed in fp32 with expf / logf after the block's position scores.
//  Score of position p: sigma_p = sum over the set's heads h (ascending) of
//  (l[h,row0,p] + l[h,row1,p]) in that fixed fp32 order; -0 is taken as +0.  Ties
//  at the k-th place go to the smaller index; output is ascending.  With n collected
//  rows the head term is (((l0 + l1) + l2) + ...); with softmax weights (Sparse
//  Glimpse page, "Core claim": per-head attention weights of the last verification
//  queries) it is the same sum of exp(l[h,c,p] - lse[h,row_c]).
//
// How
//  * score_kernel streams the two logit rows of every head once (the only HBM-
//    sized read), writes an order-preserving uint32 key per item, and builds a
//    4096-bin histogram of the top 12 key bits in LDS, flushed with one global
//    atomic per non-empty bin.  A workgroup covers one to eight 512-position chunks,
//    as many as still leave four workgroups per CU, so that large calls clear and
//    flush fewer histograms.
//  * No clearing pass: the previous call's finish_kernel left the histograms clean and
//    wrote a marker for its layout; collect trusts them only if the marker matches and
//    the counts add up to the pool, and rebuilds them from the keys otherwise.
//  * collect_kernel finds the bin that holds the k-th item, counts the items above
//    it per 4096-item chunk and appends the bin's items as 44-bit composites
//    (20 low key bits, then the complemented index) to a candidate list; each
//    thread owns 4 to 16 consecutive items (1024 to 256 threads, as many as the
//    chunks' workgroups leave per CU), and one scan places a workgroup's appends.
//  * finish_kernel (one workgroup per chunk) loads the candidates into LDS and
//    radix-selects the exact boundary composite in up to four 11-bit passes,
//    stopping once the chosen digit holds a single candidate.  Every chunk does this
//    itself, which costs less than a separate launch.  It then derives its output
//    offset from the earlier chunks' counts and candidates, and writes its kept
//    items in ascending order with a workgroup prefix sum.
//  With logit sums no transcendental function and no multiply is involved, so the
//  result is bit-identical to the same rule evaluated on the CPU in the same order;
//  softmax weights go through expf and match the CPU rule to within its rounding.
#include "lcs_internal.h"

namespace lcs {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kItemBits = 24;                       // items < 2^24
constexpr uint32_t kItemMask = (1u << kItemBits) - 1;

__device__ __forceinline__ uint32_t f2key(float f) {
  uint32_t u = __float_as_uint(f);
  if (f == 0.f) u = 0u;                             // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t composite(uint32_t key, int item) {
  return ((uint64_t)(key & 0xFFFFFu) << kItemBits) | (uint64_t)(kItemMask - (uint32_t)item);
}

struct Win {
  int L, n, lo, hi;
  bool all;
};

// Items, pool [lo, hi) and the keep-everything case for sequence b.
__device__ __forceinline__ Win window(const SelArgs& a, int b) {
  Win w;
  w.L = min(max(a.prefix_len[b], 0), a.max_len);
  if (a.mode == LCS_SEL_BLOCK) {
    const int bs = 1 << a.lg_bs;
    w.n = (w.L + bs - 1) >> a.lg_bs;
    w.lo = (a.n_sink + bs - 1) >> a.lg_bs;
    w.hi = (a.n_recent > 0) ? ((w.L - a.n_recent) >= 0 ? (w.L - a.n_recent) >> a.lg_bs : -1) : w.n;
    w.all = (w.lo >= w.hi) || (w.hi - w.lo <= a.top_k);
  } else {
    w.n = w.L;
    w.lo = a.n_sink;
    w.hi = w.L - a.n_recent;
    w.all = w.L <= a.n_sink + a.top_k + a.n_recent;
  }
  return w;
}

// A value that no kernel of the call writes while this one runs, read through the
// constant address space: a scalar load (one per wave, through the scalar cache) where a
// global read of one address by every thread would send every wave's request to it.
template <typename T>
__device__ __forceinline__ T ld_uniform(const T* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}

// Block-wide exclusive prefix sum over NT threads (NT a multiple of 64).
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* s_wave, uint32_t& total) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const uint32_t x = wave_incl_scan(v);
  if (lane == 63) s_wave[w] = x;
  __syncthreads();
  uint32_t pre = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const uint32_t t = s_wave[i];
    pre += (i < w) ? t : 0u;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return pre + x - v;
}

// the N keys of items [i0, i0 + N) (N = 4, 8 or 16); i0 is a multiple of N below
// item_cap, which is a multiple of 16, so the 16-byte loads stay inside the set's keys
template <int N>
__device__ __forceinline__ void load_keys(const uint32_t* keys, int i0, uint32_t (&k)[N]) {
#pragma unroll
  for (int v = 0; v < N / 4; ++v) {
    const uint4 x = *reinterpret_cast<const uint4*>(keys + i0 + 4 * v);
    k[4 * v] = x.x;
    k[4 * v + 1] = x.y;
    k[4 * v + 2] = x.z;
    k[4 * v + 3] = x.w;
  }
}


// Score of one head's rows at positions p, p + 1 (both < L when BOTH), into t0, t1.
// NR2: exactly two rows (the Collect-2-Query layout), summed as one pair.
template <int KIND, bool NR2, bool BOTH>
__device__ __forceinline__ void head_score(const SelArgs& a, const float* hb, int b, int h, float& t0, float& t1) {
  const int nr = NR2 ? 2 : a.n_rows;
  if (KIND == SCORE_LOGIT_SUM) {
    if (BOTH) {
      // each logit is read once per call: non-temporal loads (128K x 8: 71.9 -> 68.5 us)
      f32x2 x = __builtin_nontemporal_load(reinterpret_cast<const f32x2*>(hb));
      t0 = x.x;
      t1 = x.y;
      for (int c = 1; c < nr; ++c) {
        x = __builtin_nontemporal_load(reinterpret_cast<const f32x2*>(hb + (size_t)c * a.ld));
        t0 = t0 + x.x;
        t1 = t1 + x.y;
      }
    } else {
      t0 = hb[0];
      for (int c = 1; c < nr; ++c) t0 = t0 + hb[(size_t)c * a.ld];
      t1 = 0.f;
    }
  } else {
    uint64_t rm = a.rows_mask;
    t0 = t1 = 0.f;
    for (int c = 0; c < nr; ++c) {
      const int row = __builtin_ctzll(rm);
      rm &= rm - 1;
      const float ls = a.lse[((size_t)b * a.n_q + row) * a.Hq + h];
      const float* rp = hb + (size_t)c * a.ld;
      t0 = t0 + expf(rp[0] - ls);
      if (BOTH) t1 = t1 + expf(rp[1] - ls);
    }
  }
}

// sigma, keys and the first-digit histogram for kScorePos positions of one set.
// IT > 1 (logit sums of two rows, or of one row per head as for partial scores; IT =
// score_iters): when the workgroup's IT chunks lie wholly in the prefix, the loop runs
// heads outer and chunks inner, so that every chunk's loads of a head batch are in
// flight together, one round trip per batch instead of one per chunk and batch; each
// position still sums its heads in ascending order (64K x 4 per-KV-head sets, 4 chunks
// of 5 heads: select 42.3 -> 38.8 us; 128K x 8: 65.2 -> 64.7 us; with one chunk per
// workgroup the per-chunk loop is kept, 0.3 us faster at 32K).
template <int KIND, bool NR2, int IT = 0>
__global__ void __launch_bounds__(256) score_kernel(SelArgs a) {
  const int set = blockIdx.y;
  const int b = set / a.n_sets;
  const int s = set - b * a.n_sets;
  const Win w = window(a, b);
  if (w.all || a.top_k == 0) return;
  if (blockIdx.x == 0 && threadIdx.x == 0) a.cand_count[set] = 0;   // collect appends after this launch
  // a workgroup covers score_iters consecutive kScorePos-position chunks (one in block
  // mode) and flushes its histogram once
  const int iters = (a.mode == LCS_SEL_BLOCK) ? 1 : a.score_iters;
  int iters_done = 0;
  const int pbase = blockIdx.x * iters * kScorePos;
  if (pbase >= w.L) return;
  const int tid = threadIdx.x;
  const int h0 = (a.mode == LCS_SEL_SHARED) ? 0 : s * a.G;
  const int nh = (a.mode == LCS_SEL_SHARED) ? a.Hq : a.G;

  __shared__ uint32_t lh[kHistBins];
  __shared__ uint32_t bm[kScorePos / 4];
  __shared__ float sg[kScorePos];      // block log-sum-exp: the workgroup's position scores
  for (int i = tid; i < kHistBins; i += 256) lh[i] = 0;
  if (a.mode == LCS_SEL_BLOCK)
    for (int i = tid; i < kScorePos / 4; i += 256) bm[i] = 0;
  __syncthreads();

  uint32_t* keys = a.keys + (size_t)set * a.item_cap;
  if constexpr (IT > 0 && KIND == SCORE_LOGIT_SUM) {
    // two rows per head (NR2), or one (partial scores: one row per KV head)
    constexpr int NR = NR2 ? 2 : 1;
    if ((NR2 || a.n_rows == 1) && a.mode != LCS_SEL_BLOCK && a.vec4 && pbase + IT * kScorePos <= w.L) {
      const float* base = a.logits + (size_t)b * a.Hq * NR * a.ld + pbase + 2 * tid;
      float acc0[IT], acc1[IT];
#pragma unroll
      for (int it = 0; it < IT; ++it) acc0[it] = acc1[it] = 0.f;
      constexpr int kHU = IT * NR >= 32 ? 1 : 32 / (IT * NR);   // heads per batch: 32 loads in flight
#pragma unroll kHU
      for (int hh = 0; hh < nh; ++hh) {
        const float* hb = base + (size_t)(h0 + hh) * NR * a.ld;
        f32x2 x0[IT], x1[IT];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
          x0[it] = __builtin_nontemporal_load(reinterpret_cast<const f32x2*>(hb + it * kScorePos));
          if constexpr (NR2)
            x1[it] = __builtin_nontemporal_load(reinterpret_cast<const f32x2*>(hb + a.ld + it * kScorePos));
        }
#pragma unroll
        for (int it = 0; it < IT; ++it) {
          if constexpr (NR2) {
            acc0[it] = acc0[it] + (x0[it].x + x1[it].x);
            acc1[it] = acc1[it] + (x0[it].y + x1[it].y);
          } else {
            acc0[it] = acc0[it] + x0[it].x;
            acc1[it] = acc1[it] + x0[it].y;
          }
        }
      }
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        const int p = pbase + it * kScorePos + 2 * tid;
        const uint32_t k0 = f2key(acc0[it]), k1 = f2key(acc1[it]);
        *reinterpret_cast<uint2*>(keys + p) = make_uint2(k0, k1);
        if (p >= w.lo && p < w.hi) atomicAdd(&lh[k0 >> 20], 1u);
        if (p + 1 >= w.lo && p + 1 < w.hi) atomicAdd(&lh[k1 >> 20], 1u);
      }
      iters_done = IT;
    }
  }
  for (int it = iters_done; it < iters; ++it) {
    const int p0 = pbase + it * kScorePos;
    if (p0 >= w.L) break;
    const int p = p0 + 2 * tid;          // this thread's two positions
    float acc0 = 0.f, acc1 = 0.f;
    const int nr = NR2 ? 2 : a.n_rows;
    const float* base = a.logits + (size_t)b * a.Hq * nr * a.ld;
    if (a.vec4 && p + 1 < w.L) {
#pragma unroll 8
      for (int hh = 0; hh < nh; ++hh) {
        float t0, t1;
        head_score<KIND, NR2, true>(a, base + (size_t)(h0 + hh) * nr * a.ld + p, b, h0 + hh, t0, t1);
        acc0 = acc0 + t0;
        acc1 = acc1 + t1;
      }
    } else if (p < w.L) {
      for (int hh = 0; hh < nh; ++hh) {
        const float* hb = base + (size_t)(h0 + hh) * nr * a.ld + p;
        float t0, t1, u0, u1;
        head_score<KIND, NR2, false>(a, hb, b, h0 + hh, t0, t1);
        acc0 = acc0 + t0;
        if (p + 1 < w.L) {
          head_score<KIND, NR2, false>(a, hb + 1, b, h0 + hh, u0, u1);
          acc1 = acc1 + u0;
        }
      }
    }
    const uint32_t k0 = f2key(acc0), k1 = f2key(acc1);
    if (a.mode != LCS_SEL_BLOCK) {
      if (p + 1 < w.L) {
        *reinterpret_cast<uint2*>(keys + p) = make_uint2(k0, k1);
      } else if (p < w.L) {
        keys[p] = k0;
      }
      if (p >= w.lo && p < w.hi) atomicAdd(&lh[k0 >> 20], 1u);
      if (p + 1 >= w.lo && p + 1 < w.hi) atomicAdd(&lh[k1 >> 20], 1u);
    } else if (!a.block_lse) {
      if (p < w.L) atomicMax(&bm[(2 * tid) >> a.lg_bs], k0);
      if (p + 1 < w.L) atomicMax(&bm[(2 * tid + 1) >> a.lg_bs], k1);
    } else {
      sg[2 * tid] = acc0;
      sg[2 * tid + 1] = acc1;
    }
  }
  __syncthreads();
  if (a.mode == LCS_SEL_BLOCK) {
    const int bs = 1 << a.lg_bs;
    const int nbc = kScorePos >> a.lg_bs;
    const int c0 = pbase >> a.lg_bs;
    for (int cl = tid; cl < nbc; cl += 256) {
      const int c = c0 + cl;
      if (c < w.n) {
        uint32_t key = bm[cl];
        if (a.block_lse) {
          // log-sum-exp of the block's prefix positions, shifted by their max
          const int n = min(bs, w.L - c * bs);
          const float* x = sg + cl * bs;
          float m = -INFINITY;
          for (int t = 0; t < n; ++t) m = fmaxf(m, x[t]);
          float z = 0.f;
          for (int t = 0; t < n; ++t) z += expf(x[t] - m);
          key = f2key(m + logf(z));
        }
        keys[c] = key;
        if (c >= w.lo && c < w.hi) atomicAdd(&lh[key >> 20], 1u);
      }
    }
    __syncthreads();
  }
  // flush: every bin count of this thread is read from LDS first (one round trip), then
  // the non-empty ones go out as atomics (a loop of read, wait, atomic waits 16 times)
  uint32_t* gh = a.hist + (size_t)set * kHistBins;
  constexpr int kFlush = kHistBins / 256;
  uint32_t hv[kFlush];
#pragma unroll
  for (int k = 0; k < kFlush; ++k) hv[k] = lh[tid + 256 * k];
#pragma unroll
  for (int k = 0; k < kFlush; ++k)
    if (hv[k]) atomicAdd(&gh[tid + 256 * k], hv[k]);
}

// Threshold bin of a set from its histogram: the bin holding the k-th largest item.
// CT threads, each owning kHistBins / CT consecutive bins.
template <int CT>
__device__ uint32_t find_bin(const SelArgs& a, const uint32_t* h, uint32_t* s_wave, int* sh_bin,
                             uint32_t* sh_above) {
  constexpr int BPT = kHistBins / CT;
  const int tid = threadIdx.x;
  uint32_t hv[BPT];
  uint32_t c = 0;
#pragma unroll
  for (int e = 0; e < BPT; ++e) {
    hv[e] = h[BPT * tid + e];
    c += hv[e];
  }
  uint32_t total;
  const uint32_t excl = block_excl_scan<CT>(c, s_wave, total);
  const uint32_t K = (uint32_t)a.top_k;
  const uint32_t above_t = total - excl - c;       // items in bins above this thread's range
  if (above_t < K && above_t + c >= K) {
    uint32_t cum = above_t;
    for (int e = BPT - 1; e >= 0; --e) {
      if (cum + hv[e] >= K) {
        *sh_bin = BPT * tid + e;
        *sh_above = cum;
        break;
      }
      cum += hv[e];
    }
  }
  __syncthreads();
  return total;
}

// CT threads (1024, 512 or 256, as the finish pass), each owning kItemChunk / CT items
template <int CT>
__global__ void __launch_bounds__(CT) collect_kernel(SelArgs a) {
  constexpr int kIPT = kItemChunk / CT;
  const int set = blockIdx.y;
  const int b = set / a.n_sets;
  const Win w = window(a, b);
  if (w.all || a.top_k == 0) return;
  const int tid = threadIdx.x;
  __shared__ uint32_t s_wave[CT / 64];
  __shared__ int sh_bin;
  __shared__ uint32_t sh_above, lqbase;
  if (tid == 0) {
    sh_bin = 0;
    sh_above = 0;
  }
  // the marker is read first, so that its check after the scan costs no round trip
  // (as a relaxed atomic load, which the compiler does not sink past the barriers to its use)
  const uint64_t marker = __hip_atomic_load(a.marker, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // this thread's kIPT consecutive keys do not depend on the bin: they load while the
  // histogram is scanned
  const int i0 = blockIdx.x * kItemChunk + kIPT * tid;
  const bool mine = i0 < w.hi && i0 + kIPT > w.lo;
  uint32_t k[kIPT], flags = 0, n_above = 0;
  const uint32_t* keys = a.keys + (size_t)set * a.item_cap;
  if (mine) load_keys<kIPT>(keys, i0, k);
  __syncthreads();
  // The global histogram is valid when the last call of this layout left it clean (its
  // finish pass zeroed it and wrote the marker) and it counts exactly the pool's items.
  // Otherwise (a fresh or reused workspace) every workgroup rebuilds the set's histogram
  // from the keys in LDS; the finish pass then leaves it clean for the next call.
  const uint32_t h_total = find_bin<CT>(a, a.hist + (size_t)set * kHistBins, s_wave, &sh_bin, &sh_above);
  if (marker != a.marker_value || h_total != (uint32_t)(w.hi - w.lo)) {
    __shared__ uint32_t lhist[kHistBins];
    for (int i = tid; i < kHistBins; i += CT) lhist[i] = 0;
    if (tid == 0) {
      sh_bin = 0;
      sh_above = 0;
    }
    __syncthreads();
    // the pool's keys in 16-byte groups, kRebuildLoads groups in flight per thread; a
    // group ends at or below item_cap (a multiple of 16 and at least the item count).
    // Groups past the pool load the last group again (unconditional loads stay in
    // flight together) and count nothing.
    constexpr int kRebuildLoads = 8;
    const int q0 = w.lo >> 2, q1 = (w.hi + 3) >> 2;
    for (int q = q0 + tid; q < q1; q += kRebuildLoads * CT) {
      uint4 x[kRebuildLoads];
#pragma unroll
      for (int u = 0; u < kRebuildLoads; ++u)
        x[u] = *reinterpret_cast<const uint4*>(keys + 4 * min(q + CT * u, q1 - 1));
#pragma unroll
      for (int u = 0; u < kRebuildLoads; ++u) {
        const int it = 4 * (q + CT * u);      // past the pool when the group was clamped
        const uint32_t kv[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (it + e >= w.lo && it + e < w.hi) atomicAdd(&lhist[kv[e] >> 20], 1u);
      }
    }
    __syncthreads();
    find_bin<CT>(a, lhist, s_wave, &sh_bin, &sh_above);
  }
  const int bin = sh_bin;
  if (blockIdx.x == 0 && tid == 0) {
    a.thr[(size_t)set * 2 + 0] = (uint64_t)bin;
    a.thr[(size_t)set * 2 + 1] = (uint64_t)sh_above;
  }
  // count the items above the bin, flag the bin's (branch-free, as in the finish pass)
  if (mine) {
#pragma unroll
    for (int e = 0; e < kIPT; ++e) {
      const bool in = (i0 + e >= w.lo) & (i0 + e < w.hi);
      const uint32_t dg = k[e] >> 20;
      n_above += (uint32_t)(in & (dg > (uint32_t)bin));
      flags |= (uint32_t)(in & (dg == (uint32_t)bin)) << e;
    }
  }
  // one scan of (above << 16 | candidates); both are at most kItemChunk per workgroup
  uint32_t total;
  const uint32_t excl = block_excl_scan<CT>((n_above << 16) | __builtin_popcount(flags), s_wave, total);
  if (tid == 0) {
    lqbase = (total & 0xFFFFu) ? atomicAdd(&a.cand_count[set], total & 0xFFFFu) : 0u;
    a.chunk_above[(size_t)set * a.n_chunks + blockIdx.x] = total >> 16;
  }
  __syncthreads();
  uint64_t* cand = a.cand + (size_t)set * a.item_cap;
  uint32_t pos = lqbase + (excl & 0xFFFFu);
#pragma unroll
  for (int e = 0; e < kIPT; ++e) {
    const uint32_t f = (flags >> e) & 1u;
    if (f && pos < (uint32_t)a.item_cap) cand[pos] = composite(k[e], i0 + e);
    pos += f;
  }
}

// The id written for item it of sequence b: the position, or its physical slot.
__device__ __forceinline__ int32_t emit_id(const SelArgs& a, int b, int it) {
  if (a.bt == nullptr) return it;
  const int32_t page = a.bt[(size_t)b * a.max_pages + (it >> a.lg_page)];
  return (page << a.lg_page) | (it & ((1 << a.lg_page) - 1));
}

constexpr int kFinLDS = 8192;      // candidates a workgroup holds in LDS
constexpr int kMaxScoreIters = 8;  // most kScorePos chunks one score workgroup covers
constexpr long long kScoreWGsPerCU = 4;   // score workgroups per CU to keep
constexpr int kManyReads = 16;             // values read per position that need all four

// Boundary and output of one 4096-item chunk (one workgroup per chunk and set).  Every
// chunk's workgroup finds the exact boundary composite itself: the radix passes over
// the first-digit bin's candidates cost less than one more launch.  It then places its
// kept items after the sink window, the kept items of the chunks before it (their items
// above the bin, counted by collect, and their candidates at or above the boundary) and
// the kept items before it in this chunk.  FT threads: 1024 when the chunks of all sets
// fit in one round of the CUs, 512 when they fit with two workgroups per CU (the LDS
// holds two), else 256: fewer waves make the radix passes' barriers cheaper when several
// workgroups share a CU, more threads take fewer items each (measured at 64K x 4
// per-KV-head sets, 512 workgroups: select 52.7 us with 1024, 50.2 with 256, and with
// 512 threads 44.7 -> 42.8 us on the current passes; 128K x 8 and 32K run 1024).
template <int FT>
__global__ void __launch_bounds__(FT) finish_kernel(SelArgs a) {
  constexpr int kFinThreads = FT;
  constexpr int kFinIPT = kItemChunk / FT;   // consecutive items per thread
  constexpr int kFinBPT = 2048 / FT;         // radix bins per thread in a pass
  const int set = blockIdx.y;
  const int b = set / a.n_sets;
  const Win w = window(a, b);
  const int tid = threadIdx.x;
  const int c0 = blockIdx.x * kItemChunk;          // first item of this chunk
  int32_t* out = a.indices + (size_t)set * a.cap;
  // the histograms were read by collect: leave them clean for the next call of this
  // layout, which then needs no clearing pass (the marker says they are clean)
  if (blockIdx.x == 0) {
    uint32_t* gh = a.hist + (size_t)set * kHistBins;
    for (int i = tid; i < kHistBins; i += kFinThreads) gh[i] = 0u;
    if (set == 0 && tid == 0) *a.marker = a.marker_value;
  }
  if (w.all) {
    for (int it = c0 + tid; it < min(w.n, c0 + kItemChunk); it += kFinThreads)
      if (it < a.cap) out[it] = emit_id(a, b, it);
    if (blockIdx.x == 0 && tid == 0) a.counts[set] = min(w.n, a.cap);
    return;
  }
  const int K = a.top_k;
  __shared__ uint64_t lc[kFinLDS];
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t s_wave[kFinThreads / 64];
  __shared__ uint64_t sh_prefix, sh_one;
  __shared__ uint32_t sh_rem, sh_cnt;
  // this thread's kFinIPT consecutive items (t0 is a multiple of 4 below item_cap, a
  // multiple of 16, so the 16-byte loads stay inside the set's keys); they do not depend
  // on the boundary, so they are loaded first
  const int t0 = c0 + kFinIPT * tid;
  uint32_t kk[kFinIPT];
#pragma unroll
  for (int e = 0; e < kFinIPT; ++e) kk[e] = 0u;
  if (K > 0 && t0 < w.hi && t0 + kFinIPT > w.lo) {
#pragma unroll
    for (int v = 0; v < kFinIPT / 4; ++v) {
      const uint4 q = *reinterpret_cast<const uint4*>(a.keys + (size_t)set * a.item_cap + t0 + 4 * v);
      kk[4 * v] = q.x;
      kk[4 * v + 1] = q.y;
      kk[4 * v + 2] = q.z;
      kk[4 * v + 3] = q.w;
    }
  }
  // Loaded with the keys, before anything that depends on them: the earlier chunks'
  // above-bin counts, and the first kSpec * FT candidates (read before their count is
  // known; entries past the count are left unused), so that the candidates' count and
  // the chunks' offsets add no round trip of their own.
  constexpr int kSpec = 1024 / FT;
  const uint64_t* gcand = a.cand + (size_t)set * a.item_cap;
  const uint32_t* cabove = a.chunk_above + (size_t)set * a.n_chunks;
  uint32_t part = 0;
  uint64_t spec[kSpec], thr_bin = 0, thr_above = 0;
  int n_cand = 0;
  if (K > 0) {
#pragma unroll
    for (int u = 0; u < kSpec; ++u) {
      const int e = tid + u * kFinThreads;
      spec[u] = (e < a.item_cap) ? gcand[e] : 0ull;
    }
    thr_bin = ld_uniform(a.thr + (size_t)set * 2 + 0);
    thr_above = ld_uniform(a.thr + (size_t)set * 2 + 1);
    n_cand = (int)ld_uniform(a.cand_count + set);
    if (tid < (int)blockIdx.x) part = cabove[tid];
    for (int c = tid + kFinThreads; c < (int)blockIdx.x; c += kFinThreads) part += cabove[c];
  }
  int bin = 0;
  uint64_t cstar = ~0ull;
  uint32_t base = (uint32_t)w.lo;
  if (K > 0) {
    bin = (int)thr_bin;
    const uint32_t above = (uint32_t)thr_above;
    const int n_c = min(n_cand, a.item_cap);
    const bool in_lds = n_c <= kFinLDS;
    if (in_lds) {
#pragma unroll
      for (int u = 0; u < kSpec; ++u) {
        const int e = tid + u * kFinThreads;
        if (e < n_c) lc[e] = spec[u];
      }
      for (int e = tid + kSpec * kFinThreads; e < n_c; e += kFinThreads) lc[e] = gcand[e];
    }
    const uint64_t* cand = in_lds ? lc : gcand;
    if (tid == 0) {
      sh_prefix = 0;
      sh_rem = (uint32_t)K - above;
    }
    __syncthreads();
    // the sh_rem-th largest candidate composite, 11 bits per pass; stop as soon as the
    // chosen digit holds a single candidate
    uint64_t mask = 0;
    int pass = 0;
    for (; pass < 4; ++pass) {
      const int shift = 33 - 11 * pass;
      for (int i = tid; i < 2048; i += kFinThreads) hist[i] = 0;
      __syncthreads();
      const uint64_t prefix = sh_prefix;
      const uint32_t rem = sh_rem;
      for (int e = tid; e < n_c; e += kFinThreads) {
        const uint64_t cv = cand[e];
        if ((cv & mask) == prefix) atomicAdd(&hist[(cv >> shift) & 2047u], 1u);
      }
      __syncthreads();
      // the digit holding the rem-th largest remaining composite (suffix sums over bins):
      // this thread owns bins [kFinBPT * tid, kFinBPT * tid + kFinBPT)
      uint32_t hv[kFinBPT], c = 0;
#pragma unroll
      for (int e = 0; e < kFinBPT; ++e) {
        hv[e] = hist[kFinBPT * tid + e];
        c += hv[e];
      }
      uint32_t total;
      const uint32_t excl = block_excl_scan<kFinThreads>(c, s_wave, total);
      const uint32_t above_t = total - excl - c;
      if (above_t < rem && above_t + c >= rem) {
        uint32_t cum = above_t;
#pragma unroll
        for (int e = kFinBPT - 1; e >= 0; --e) {
          if (cum + hv[e] >= rem) {
            sh_prefix = prefix | ((uint64_t)(kFinBPT * tid + e) << shift);
            sh_rem = rem - cum;
            sh_cnt = hv[e];
            break;
          }
          cum += hv[e];
        }
      }
      mask |= (uint64_t)2047u << shift;
      __syncthreads();
      if (sh_cnt == 1) break;
    }
    cstar = sh_prefix;
    if (pass < 3) {                 // one candidate carries the chosen prefix: it is the answer
      const uint64_t prefix = sh_prefix;
      for (int e = tid; e < n_c; e += kFinThreads) {
        const uint64_t cv = cand[e];
        if ((cv & mask) == prefix) sh_one = cv;
      }
      __syncthreads();
      cstar = sh_one;
    }
    // kept items of the chunks before this one: their items above the bin (part, loaded
    // above) and their candidates at or above the boundary
    for (int e = tid; e < n_c; e += kFinThreads) {
      const uint64_t cv = cand[e];
      const int item = (int)(kItemMask - (uint32_t)(cv & kItemMask));
      part += (cv >= cstar && item < c0) ? 1u : 0u;
    }
    uint32_t before;
    block_excl_scan<kFinThreads>(part, s_wave, before);
    base += before;
  }
  // Both loops below are branch-free up to the store: this code runs once per workgroup,
  // and every taken branch of a one-shot path costs an instruction fetch.
  uint32_t flags = 0, cnt = 0;
  if (K > 0) {
#pragma unroll
    for (int e = 0; e < kFinIPT; ++e) {
      const int it = t0 + e;
      const uint32_t dg = kk[e] >> 20;
      // kept: in the pool, and above the boundary composite
      const bool keep = (it >= w.lo) & (it < w.hi) &
                        ((dg > (uint32_t)bin) | ((dg == (uint32_t)bin) & (composite(kk[e], it) >= cstar)));
      flags |= (uint32_t)keep << e;
      cnt += (uint32_t)keep;
    }
  }
  uint32_t total;
  uint32_t pos = base + block_excl_scan<kFinThreads>(cnt, s_wave, total);
  // output slot of each item (-1: none): a sink item keeps its position, a recent item
  // follows the K kept pool items, and kept pool items take consecutive slots
  const int rbase = w.lo + K - w.hi;
#pragma unroll
  for (int e = 0; e < kFinIPT; ++e) {
    const int it = t0 + e;
    const uint32_t kept = (flags >> e) & 1u;
    int o = kept ? (int)pos : -1;
    o = (it < w.lo) ? it : o;
    o = (it >= w.hi) ? rbase + it : o;
    o = (it < w.n) ? o : -1;
    pos += kept;
    if (o >= 0 && o < a.cap) out[o] = emit_id(a, b, it);
  }
  if (blockIdx.x == 0 && tid == 0) a.counts[set] = min(w.lo + K + (w.n - w.hi), a.cap);
}

}  // namespace

SelPlan select_plan(int32_t B, int32_t Hq, int32_t Hkv, int32_t mode, int32_t max_len,
                    int32_t block_size, int32_t cus, int32_t reads) {
  SelPlan p{};
  p.n_sets = (mode == LCS_SEL_SHARED) ? 1 : Hkv;
  const size_t NS = (size_t)B * p.n_sets;
  long long items = max_len;
  if (mode == LCS_SEL_BLOCK) items = (max_len + block_size - 1) / block_size;
  if (items < 1) items = 1;
  p.item_cap = (int32_t)align_up((size_t)items, 16);
  p.n_chunks = (int32_t)((items + kItemChunk - 1) / kItemChunk);
  // score workgroups: several chunks each while that still leaves kScoreWGsPerCU
  // workgroups per CU (fewer histogram clears and flushes); a set whose positions read
  // few values (partial scores, small groups) keeps half as many, each covering more
  // chunks (measured: partial scores at 64K x 4, 28.1 -> 26.7 us; at 128K x 8, 28.2 ->
  // 27.4 us; two logit rows of 32 heads at 128K x 8 need the four: 64.2 against 65.4)
  const long long pos_chunks = ((long long)(max_len > 0 ? max_len : 1) + kScorePos - 1) / kScorePos;
  const long long ncu = cus > 0 ? cus : kDefaultCUs;
  p.score_iters = 1;
  if (mode != LCS_SEL_BLOCK)
    while (p.score_iters < kMaxScoreIters &&
           pos_chunks * (long long)NS / (2 * p.score_iters) >=
               (reads > 0 && reads < kManyReads ? kScoreWGsPerCU / 2 : kScoreWGsPerCU) * ncu)
      p.score_iters *= 2;
  p.n_pos_chunks = (int32_t)((pos_chunks + p.score_iters - 1) / p.score_iters);
  {
    const long long wg = (long long)p.n_chunks * (long long)NS, nc = cus > 0 ? cus : kDefaultCUs;
    p.fin_threads = wg <= nc ? 1024 : (wg <= 2 * nc ? 512 : 256);
  }
  p.keys_bytes = align_up(NS * p.item_cap * 4, 256);
  p.hist_bytes = align_up(NS * kHistBins * 4, 256);
  p.cc_bytes = align_up(NS * 4, 256);
  p.cand_bytes = align_up(NS * p.item_cap * 8, 256);
  p.ca_bytes = align_up(NS * p.n_chunks * 4, 256);
  p.thr_bytes = align_up(NS * 2 * 8, 256);
  p.mk_bytes = 256;
  p.total_bytes = p.keys_bytes + p.hist_bytes + p.cc_bytes + p.cand_bytes + p.ca_bytes +
                  p.thr_bytes + p.mk_bytes;
  return p;
}

hipError_t select_launch(const SelPlan& p, SelArgs a, void* workspace, hipStream_t stream) {
  char* ws = static_cast<char*>(workspace);
  a.keys = reinterpret_cast<uint32_t*>(ws); ws += p.keys_bytes;
  a.hist = reinterpret_cast<uint32_t*>(ws); ws += p.hist_bytes;
  a.cand_count = reinterpret_cast<uint32_t*>(ws); ws += p.cc_bytes;
  a.cand = reinterpret_cast<uint64_t*>(ws); ws += p.cand_bytes;
  a.chunk_above = reinterpret_cast<uint32_t*>(ws); ws += p.ca_bytes;
  a.thr = reinterpret_cast<uint64_t*>(ws); ws += p.thr_bytes;
  a.marker = reinterpret_cast<uint64_t*>(ws);
  a.n_sets = p.n_sets;
  a.item_cap = p.item_cap;
  a.n_chunks = p.n_chunks;
  a.n_pos_chunks = p.n_pos_chunks;
  a.score_iters = p.score_iters;
  const int NS = a.B * p.n_sets;
  // layout-specific, so that a workspace last used with another layout is not trusted
  a.marker_value = 0x9E3779B97F4A7C15ull ^ ((uint64_t)NS << 40) ^ ((uint64_t)p.item_cap << 8) ^
                   (uint64_t)p.n_chunks;
  hipError_t e;
  const dim3 sgrid(p.n_pos_chunks, NS);
  if (a.kind == SCORE_SOFTMAX_WT)
    hipLaunchKernelGGL((score_kernel<SCORE_SOFTMAX_WT, false>), sgrid, dim3(256), 0, stream, a);
  else if (a.n_rows == 2 && p.score_iters == 2)
    hipLaunchKernelGGL((score_kernel<SCORE_LOGIT_SUM, true, 2>), sgrid, dim3(256), 0, stream, a);
  else if (a.n_rows == 2 && p.score_iters == 4)
    hipLaunchKernelGGL((score_kernel<SCORE_LOGIT_SUM, true, 4>), sgrid, dim3(256), 0, stream, a);
  else if (a.n_rows == 2 && p.score_iters == 8)
    hipLaunchKernelGGL((score_kernel<SCORE_LOGIT_SUM, true, 8>), sgrid, dim3(256), 0, stream, a);
  else if (a.n_rows == 2)
    hipLaunchKernelGGL((score_kernel<SCORE_LOGIT_SUM, true>), sgrid, dim3(256), 0, stream, a);
  else if (p.score_iters == 2)
    hipLaunchKernelGGL((score_kernel<SCORE_LOGIT_SUM, false, 2>), sgrid, dim3(256), 0, stream, a);
  else if (p.score_iters == 4)
    hipLaunchKernelGGL((score_kernel<SCORE_LOGIT_SUM, false, 4>), sgrid, dim3(256), 0, stream, a);
  else if (p.score_iters == 8)
    hipLaunchKernelGGL((score_kernel<SCORE_LOGIT_SUM, false, 8>), sgrid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((score_kernel<SCORE_LOGIT_SUM, false>), sgrid, dim3(256), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (p.fin_threads == 256)
    hipLaunchKernelGGL(collect_kernel<256>, dim3(p.n_chunks, NS), dim3(256), 0, stream, a);
  else if (p.fin_threads == 512)
    hipLaunchKernelGGL(collect_kernel<512>, dim3(p.n_chunks, NS), dim3(512), 0, stream, a);
  else
    hipLaunchKernelGGL(collect_kernel<1024>, dim3(p.n_chunks, NS), dim3(1024), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (p.fin_threads == 256)
    hipLaunchKernelGGL(finish_kernel<256>, dim3(p.n_chunks, NS), dim3(256), 0, stream, a);
  else if (p.fin_threads == 512)
    hipLaunchKernelGGL(finish_kernel<512>, dim3(p.n_chunks, NS), dim3(512), 0, stream, a);
  else
    hipLaunchKernelGGL(finish_kernel<1024>, dim3(p.n_chunks, NS), dim3(1024), 0, stream, a);
  return hipGetLastError();
}

}  // namespace lcs
